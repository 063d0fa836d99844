// Paged decode attention, bf16, matrix cores: one persistent, balanced pass.
//
// What is computed ("PagedAttention: Virtual Memory for the KV Cache",
// sections 1 and 13; "PagedAttention in vLLM: scattered memory, exact
// attention", sections 10-11): out[n][h] = softmax(scale * q[n][h] K^T) V over
// the S_n cached tokens of sequence n, K and V of KV head h / G gathered
// through the block table.
//
// Work decomposition
//   The work is the list of 32-token tiles of every (sequence n, KV head j)
//   "segment", segments in (n, j) order: T = Hkv * sum_n ceil(S_n / 32) tiles.
//   The launch holds exactly as many waves W as the chip keeps resident, and
//   wave w walks the tiles [w T / W, (w + 1) T / W): every wave reads the same
//   number of bytes, so all finish together and no workgroup round is left
//   half empty.  A segment that starts and ends inside one wave's range is
//   finished by that wave (output written directly).  A segment cut by range
//   boundaries leaves one (m, z, u) summary per piece; `merge_stream` combines
//   them with the common-maximum rule of the second page, section 11, in wave
//   order.
//
// Per wave, two tiles are in flight: while one tile is computed, the next
// tile's Q, keys and values and the block-table entries of the tile after it
// are loading.  One wave per SIMD (one workgroup per CU): with more, the
// oldest waves win the memory pipe and the equal split finishes unevenly.
//
// Per tile (lane = 16 gq + r), as in the partitioned kernel:
//   q.K^T  A = 16 key rows x 32 d (lane: row r, chunk 4 jj + gq, one 16-byte
//          load), B = Q^T (head r, zero for r >= G) -> S^T[4 gq + i][r]
//   P.V    A = V^T rows d = 16 mm + r, 8 tokens (4 of each 16-token slab,
//          two 8-byte loads), B = P^T: the lane's own 8 probabilities, split
//          into bf16 high and residual parts -> O^T[16 mm + 4 gq + i][r].
//
// Pool layout (per layer): K [num_blocks][Hkv][D/8][B][8], V [num_blocks][Hkv][D][B].

#include <cstdlib>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "decode_stream.h"

namespace pa {
namespace {

constexpr int kSW = 4;        // waves per workgroup
constexpr int kMaxSeqs = 3072;  // lengths and tile prefix sums live in LDS beside the stages

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

// Next tile in (n, j, ti) order; only called when one exists.
__device__ __forceinline__ TilePos advance(TilePos t, const int32_t* s_pre, int hkv) {
  if (t.ti + 1 < tiles_of(s_pre, t.n)) {
    ++t.ti;
    return t;
  }
  t.ti = 0;
  if (t.j + 1 < hkv) {
    ++t.j;
    return t;
  }
  t.j = 0;
  do {
    ++t.n;
  } while (tiles_of(s_pre, t.n) == 0);
  return t;
}

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

// Table entries of a tile's blocks.  Always loaded (index clamped into the
// row) and replaced by -1 past the end of the sequence, so no load sits behind
// a branch and the compiler can keep the pipeline's loads in flight.
template <int B, int TOK>
__device__ __forceinline__ Tb<TOK / B> load_tb(TilePos t, const int32_t* __restrict__ block_tables, int max_blocks,
                                               const int32_t* s_len) {
  const int32_t* row = block_tables + static_cast<int64_t>(t.n) * max_blocks;
  const int S = pool_tokens(s_len[t.n]);
  const int t0 = t.ti * TOK;
  Tb<TOK / B> tb;
#pragma unroll
  for (int i = 0; i < TOK / B; ++i) {
    const int e = row[min(t0 / B + i, max_blocks - 1)];
    tb.blk[i] = t0 + i * B < S ? e : -1;
  }
  return tb;
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
};

template <int D>
__device__ __forceinline__ void reset(Acc<D>& st) {
#pragma unroll
  for (int mm = 0; mm < D / 16; ++mm) st.o[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.z = 0.f;
}

typedef __attribute__((address_space(3))) unsigned char lds_byte;

// Per wave, two LDS stages for one tile's key and value block images (16 KiB
// each at D = 128).  Two distinct objects, so the compiler can tell the wait
// for one stage's copy from the other's.
constexpr int kStageBytes = 2 * 32 * 128 * 2;
__shared__ __attribute__((aligned(16))) unsigned char g_stage0[4][kStageBytes];
__shared__ __attribute__((aligned(16))) unsigned char g_stage1[4][kStageBytes];

// Bytes of one tile's keys (and, again, of its values) in LDS: the images of
// the blocks that hold its tokens -- 32 / B bf16 images of B * D * 2 bytes, or
// 64 / B FP8 images of B * D bytes.
template <int D>
constexpr int kStageHalf = 64 * D;

// Copy one tile's key and value block images into an LDS stage with
// global_load_lds (16 bytes per lane, 1 KiB per instruction, straight to LDS:
// no registers held while in flight).  A missing block (past the end, or an
// id outside the pool) is read from block 0 -- a valid address -- and its
// tokens are masked out in pv_tile.
// The tile's images lie back to back in the stage; 1 KiB piece p of them is
// one instruction, lane l bringing bytes p * 1024 + 16 l .. + 15.  An image
// smaller than 1 KiB (FP8, D = 64, B = 8: 512 bytes) shares a piece with the
// next block's image, so the lanes of one instruction read two blocks.
template <int D, int B, bool F8>
__device__ __forceinline__ void dma_tile(unsigned char* stage_ptr, int j, const Tb<kTok<F8> / B>& tb,
                                         const void* __restrict__ k_pool, const void* __restrict__ v_pool, int hkv,
                                         int num_blocks, int lane) {
  constexpr int NB = kTok<F8> / B;
  constexpr int IMG = D * B * (F8 ? 1 : 2);  // bytes of one (block, KV head) image
  constexpr int PIECES = NB * IMG / 1024;
  lds_byte* stage = (lds_byte*)stage_ptr;  // LDS address for the copy engine
  const int64_t blk_stride = static_cast<int64_t>(hkv) * IMG;
  const char* kb = reinterpret_cast<const char*>(k_pool) + static_cast<int64_t>(j) * IMG;
  const char* vb = reinterpret_cast<const char*>(v_pool) + static_cast<int64_t>(j) * IMG;
#pragma unroll
  for (int p = 0; p < PIECES; ++p) {
    int e, off;
    if constexpr (IMG >= 1024) {
      e = tb.blk[p * 1024 / IMG];
      off = p * 1024 % IMG + lane * 16;
    } else {
      constexpr int PER = 1024 / IMG;  // images per piece
      const int bi = p * PER + lane * 16 / IMG;
      e = tb.blk[p * PER];  // tb.blk[bi] by selects: a lane-dependent index would put tb in scratch
#pragma unroll
      for (int i = 1; i < PER; ++i)
        if (bi == p * PER + i) e = tb.blk[p * PER + i];
      off = lane * 16 % IMG;
    }
    const int64_t pb = (e >= 0 && e < num_blocks) ? e : 0;
    __builtin_amdgcn_global_load_lds(kb + pb * blk_stride + off, stage + p * 1024, 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb + pb * blk_stride + off, stage + kStageHalf<D> + p * 1024, 16, 0, 0);
  }
}

// Read a staged tile's MFMA operands from LDS into registers (the same lane
// roles as direct loads would give) and mark which value groups exist.
template <int D, int B>
__device__ __forceinline__ void read_tile(Buf<D>& b, const unsigned char* stage, const Tb<32 / B>& tb, int num_blocks,
                                          int r, int gq) {
  constexpr int IMG = D * B * 2;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int tk = 16 * a + r;  // key row of slab a
    const unsigned char* kimg = stage + (tk / B) * IMG + (tk % B) * 16;
#pragma unroll
    for (int jj = 0; jj < D / 32; ++jj)
      b.k[a][jj] = *reinterpret_cast<const bf16x8*>(kimg + (4 * jj + gq) * B * 16);
    const int tv = 16 * a + 4 * gq;  // first token of the value group
    const unsigned char* vimg = stage + kStageHalf<D> + (tv / B) * IMG + (tv % B) * 2;
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm) {
      const uint2 v = *reinterpret_cast<const uint2*>(vimg + (16 * mm + r) * B * 2);
      if (a == 0)
        b.v0[mm] = v;
      else
        b.v1[mm] = v;
    }
    int pv = tb.blk[0];  // tb.blk[tv / B] by selects: a lane-dependent index would put tb in scratch
#pragma unroll
    for (int i = 1; i < 32 / B; ++i)
      if (tv / B == i) pv = tb.blk[i];
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
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
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

// ---- FP8 (E4M3) cache ----------------------------------------------------------
//
// Codes are OCP E4M3; a stored code c stands for value(c) * scale, one fp32
// scale per (block, KV head) for keys and one for values.  gfx950 converts
// two codes to two bf16 in one instruction, exactly (every E4M3 value is a
// bf16 value), so both products stay bf16 x bf16 MFMAs on the codes' values
// and the scales are applied outside them: the key scale multiplies a
// token's score, the value scale its probability in P.V (the weight sum uses
// the unscaled probability).  A 64-token tile is two 32-token sub-tiles,
// each computed as a bf16 tile is.

// Register image of a staged FP8 tile for lane (r, gq).
template <int D>
struct Buf8 {
  uint4 k[2][2][D / 64];     // [sub-tile][slab] key row 16 slab + r: the 16-byte chunks of d quarter gq
  uint32_t v[2][2][D / 16];  // [sub-tile][slab][mm] value row 16 mm + r, tokens 4 gq .. 4 gq + 3 of the slab
  bool ok[2][2];             // the block of that value group is in the pool
};

// Scales of the blocks of the lane's token groups (0 where the block is missing).
struct Sc8 {
  float k[2][2], v[2][2];  // [sub-tile][slab]
};

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Eight codes (two words, lowest byte first) as eight bf16 values.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t lo, uint32_t hi) {
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Block of the lane's 4-token group that starts at tile token first + 4 gq
// (first a multiple of 16, known at compile time after unrolling).  With
// B >= 16 the 16 tokens from `first` lie in one block; with B = 8 in two,
// chosen by one select (an index computed at run time would move tb to scratch).
template <int B>
__device__ __forceinline__ int group_block(const Tb<64 / B>& tb, int first, int gq) {
  if constexpr (B >= 16)
    return tb.blk[first / B];
  else
    return gq >= 2 ? tb.blk[first / B + 1] : tb.blk[first / B];
}

template <int B>
__device__ __forceinline__ Sc8 load_scales(const Tb<64 / B>& tb, const float* __restrict__ k_scale,
                                           const float* __restrict__ v_scale, int j, int hkv, int num_blocks, int gq) {
  Sc8 sc;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int e = group_block<B>(tb, 32 * u + 16 * a, gq);
      const bool ok = e >= 0 && e < num_blocks;
      const int64_t idx = static_cast<int64_t>(ok ? e : 0) * hkv + j;
      const float kv = k_scale[idx], vv = v_scale[idx];
      sc.k[u][a] = ok ? kv : 0.f;
      sc.v[u][a] = ok ? vv : 0.f;
    }
  return sc;
}

template <int D, int B>
__device__ __forceinline__ void read_tile8(Buf8<D>& b, const unsigned char* stage, const Tb<64 / B>& tb, int num_blocks,
                                           int r, int gq) {
  constexpr int IMG = D * B;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int tk = 32 * u + 16 * a + r;  // key row
      const unsigned char* kimg = stage + (tk / B) * IMG + (tk % B) * 16;
#pragma unroll
      for (int w = 0; w < D / 64; ++w)
        b.k[u][a][w] = *reinterpret_cast<const uint4*>(kimg + (gq * (D / 64) + w) * B * 16);
      const int tv = 32 * u + 16 * a + 4 * gq;  // first token of the value group
      const unsigned char* vimg = stage + kStageHalf<D> + (tv / B) * IMG + tv % B;
#pragma unroll
      for (int mm = 0; mm < D / 16; ++mm) b.v[u][a][mm] = *reinterpret_cast<const uint32_t*>(vimg + (16 * mm + r) * B);
      const int e = group_block<B>(tb, 32 * u + 16 * a, gq);
      b.ok[u][a] = e >= 0 && e < num_blocks;
    }
}

template <int D>
__device__ __forceinline__ void qk_tile8(f32x4 (&s)[2], const uint4 (&k)[2][D / 64], const QOp<D>& qo) {
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    s[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < D / 32; ++jj) {
      const uint4 c = k[a][jj >> 1];
      const bf16x8 kop = (jj & 1) ? fp8x8_to_bf16(c.z, c.w) : fp8x8_to_bf16(c.x, c.y);
      s[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop, qo.q[jj], s[a], 0, 0, 0);
    }
  }
}

// pv_tile for one FP8 sub-tile: sk[a] = scale_log2 * key scale and sv[a] =
// value scale of the lane's token group in slab a.
template <int D>
__device__ __forceinline__ void pv_tile8(Acc<D>& st, const f32x4 (&s)[2], const uint32_t (&v)[2][D / 16],
                                         const bool (&ok)[2], int t0, int S, bool full, const float (&sk)[2],
                                         const float (&sv)[2], int gq) {
  int n0 = 4, n1 = 4;
  if (!full) {
    n0 = ok[0] ? min(max(S - (t0 + 4 * gq), 0), 4) : 0;
    n1 = ok[1] ? min(max(S - (t0 + 16 + 4 * gq), 0), 4) : 0;
  }
  float x[2][4];
  float tmax = -INFINITY;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[a][i] = i < (a ? n1 : n0) ? s[a][i] * sk[a] : -INFINITY;
      tmax = fmaxf(tmax, x[a][i]);
    }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
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
      const float pv = p * sv[a];
      const __bf16 h = static_cast<__bf16>(pv);
      phi[4 * a + i] = h;
      plo[4 * a + i] = static_cast<__bf16>(pv - static_cast<float>(h));
    }
  st.z = st.z * alpha + psum;
  if (__any(alpha != 1.f)) {
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm) st.o[mm] *= alpha;
  }
  uint32_t m0 = 0xffffffffu, m1 = 0xffffffffu;
  if (!full) {  // zero the codes of missing tokens: stale or NaN codes must not reach P.V
    m0 = n0 >= 4 ? 0xffffffffu : (1u << (8 * n0)) - 1u;
    m1 = n1 >= 4 ? 0xffffffffu : (1u << (8 * n1)) - 1u;
  }
#pragma unroll
  for (int mm = 0; mm < D / 16; ++mm) {
    const bf16x8 vop = fp8x8_to_bf16(v[0][mm] & m0, v[1][mm] & m1);
    st.o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, phi, st.o[mm], 0, 0, 0);
    st.o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, plo, st.o[mm], 0, 0, 0);
  }
}

// End of a piece of segment t: write the normalised output (whole segment) or a summary record.
template <int D>
__device__ __forceinline__ void flush(Acc<D>& st, TilePos t, bool whole, int slot, int64_t wave_id, uint16_t* out,
                                      float* rec, int hq, int g, int r, int gq) {
  float zt = st.z + __shfl_xor(st.z, 16);
  zt += __shfl_xor(zt, 32);
  if (r < g) {
    if (whole) {
      const float inv = 1.f / zt;
      uint16_t* o = out + (static_cast<int64_t>(t.n) * hq + t.j * g + r) * D + 4 * gq;
#pragma unroll
      for (int mm = 0; mm < D / 16; ++mm) {
        const uint32_t lo = f32_to_bf16_bits(st.o[mm][0] * inv) | (uint32_t(f32_to_bf16_bits(st.o[mm][1] * inv)) << 16);
        const uint32_t hi = f32_to_bf16_bits(st.o[mm][2] * inv) | (uint32_t(f32_to_bf16_bits(st.o[mm][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(o + 16 * mm) = make_uint2(lo, hi);
      }
    } else {
      float* rr = rec + (static_cast<int64_t>(wave_id * 2 + slot) * g + r) * (D + 4);
#pragma unroll
      for (int mm = 0; mm < D / 16; ++mm) *reinterpret_cast<f32x4*>(rr + 4 + 16 * mm + 4 * gq) = st.o[mm];
      if (gq == 0) {
        rr[0] = st.m;
        rr[1] = zt;
      }
    }
  }
  reset(st);
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

template <int D, int B, bool F8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void decode_stream(
    const uint16_t* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    float* __restrict__ rec, int32_t* __restrict__ prefix_out, int n_seqs, int hq, int hkv, int g, int max_blocks,
    int num_blocks, float scale_log2, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int32_t* __restrict__ slots_out, const float* __restrict__ k_scale,
    const float* __restrict__ v_scale) {
  constexpr int TOK = kTok<F8>;
  constexpr int NB = TOK / B;
  extern __shared__ int32_t sm[];
  int32_t* s_len = sm;            // [n_seqs] packed attended-token counts (pool part clamped to the table)
  int32_t* s_pre = sm + n_seqs;   // [n_seqs + 1] tile prefix sums
  __shared__ int32_t s_wsum[kSW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 15;
  const int gq = lane >> 4;

  // ---- tiles per sequence and their prefix sums (block-wide scan) ----------
  const int s_cap = max_blocks * B;
  int carry = 0;
  for (int base = 0; base < n_seqs; base += 256) {
    const int i = base + tid;
    const int S_raw = i < n_seqs ? context_lens[i] : 0;
    const int S = min(max(S_raw, 0), s_cap);
    const int hn = k_new != nullptr ? 1 : 0;  // pa_decode_step: every row attends to its new token
    const int fits = S_raw >= 0 && S_raw < s_cap ? 1 : 0;
    const int S_att = S + hn;
    int v = (S_att + TOK - 1) >> kTokShift<F8>;
#pragma unroll
    for (int dlt = 1; dlt < 64; dlt <<= 1) {
      const int u = __shfl_up(v, dlt);
      if (lane >= dlt) v += u;
    }
    if (lane == 63) s_wsum[wave] = v;
    if (i < n_seqs) s_len[i] = (S_att << 2) | (fits << 1) | hn;
    __syncthreads();
    int off = carry;
    for (int w2 = 0; w2 < wave; ++w2) off += s_wsum[w2];
    if (i < n_seqs) s_pre[i + 1] = off + v;
    carry += s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
    __syncthreads();
  }
  if (tid == 0) s_pre[0] = 0;
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = tid; i <= n_seqs; i += 256) prefix_out[i] = s_pre[i];
  // no barrier below this point: waves run independently

  Split sp;
  sp.init(static_cast<int64_t>(hkv) * s_pre[n_seqs], static_cast<int64_t>(gridDim.x) * kSW);
  // XCD-major order: workgroups are dealt to the 8 XCDs in turn (workgroup b
  // runs on XCD b % 8), so this numbering gives each XCD one contiguous share
  // of the tile list: the waves of one sequence's KV heads share that XCD's
  // L2 for Q, table rows and scales.  The merge kernel sees the same numbering.
  const int64_t wg = gridDim.x % 8 == 0 ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : blockIdx.x;
  const int64_t wave_id = wg * kSW + wave;
  const int64_t x0 = sp.start(wave_id);
  const int64_t x1 = sp.start(wave_id + 1);
  if (x0 >= x1) return;

  // locate x0: last n with hkv * s_pre[n] <= x0
  int lo = 0, hi = n_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (static_cast<int64_t>(hkv) * s_pre[mid] <= x0) lo = mid; else hi = mid - 1;
  }
  TilePos cur;
  cur.n = lo;
  {
    const int64_t rem = x0 - static_cast<int64_t>(hkv) * s_pre[lo];
    const int nt = tiles_of(s_pre, lo);
    cur.j = static_cast<int>(rem / nt);
    cur.ti = static_cast<int>(rem - static_cast<int64_t>(cur.j) * nt);
  }
  int piece_start = cur.ti;  // first tile of the current piece
  bool first_piece = true;

  Acc<D> st;
  reset(st);
  // Two LDS stages per wave: while tile x is computed (from registers read
  // out of one stage), tile x + 1's keys and values stream into the other
  // stage, its Q into registers and the table entries of tile x + 2 as well.
  // All loads are unconditional (a missing successor repeats the current
  // tile's addresses).
  QOp<D> qA, qB;
  TilePos nxt = x1 - x0 > 1 ? advance(cur, s_pre, hkv) : cur;
  Tb<NB> tbA = load_tb<B, TOK>(cur, block_tables, max_blocks, s_len);
  Tb<NB> tbB = load_tb<B, TOK>(nxt, block_tables, max_blocks, s_len);
  load_q<D, F8>(qA, cur, q, hq, g, r, gq);
  dma_tile<D, B, F8>(&g_stage0[wave][0], cur.j, tbA, k_pool, v_pool, hkv, num_blocks, lane);
  // FP8: the scales of a tile's blocks travel with it, one tile ahead like its Q
  Sc8 scA{}, scB{};
  if constexpr (F8) scA = load_scales<B>(tbA, k_scale, v_scale, cur.j, hkv, num_blocks, gq);

  int64_t x = x0;
  // One step: tile `cur` (staged in stage SC, Q in qc, blocks tbc) is computed
  // while `nxt` streams into the other stage / qn (its blocks tbn are known)
  // and the table entries of the tile after it load into tb2.  Returns false
  // after the last tile.
  // the step's new token, for tiles that end a segment holding one
  auto wants_new = [&](TilePos t) -> bool {
    return !F8 && k_new != nullptr && has_new_token(s_len[t.n]) && t.ti == tiles_of(s_pre, t.n) - 1;
  };
  // one buffer: a step patches its tile before it loads the next tile's token
  NewTok<D> ntok;
  if (wants_new(cur)) load_new<D>(ntok, cur, k_new, v_new, slots, hkv, r, gq);
  auto step = [&](auto sc_tag, QOp<D>& qc, const Tb<NB>& tbc, const Sc8& scc, QOp<D>& qn, const Tb<NB>& tbn,
                  Sc8& scn, Tb<NB>& tb2) -> bool {
    constexpr int SC = decltype(sc_tag)::value;
    unsigned char(&stc)[4][kStageBytes] = SC == 0 ? g_stage0 : g_stage1;
    unsigned char(&stn)[4][kStageBytes] = SC == 0 ? g_stage1 : g_stage0;
    // The compiler orders any LDS read after every outstanding LDS copy, so the
    // current stage is read into registers first; the next tile's copies are
    // issued after it and stay in flight through this tile's compute.
    const bool has_next = x + 1 < x1;
    const int packed = s_len[cur.n];
    const int S = attended_tokens(packed);
    const int nt_cur = tiles_of(s_pre, cur.n);
    const TilePos nxt2 = x + 2 < x1 ? advance(nxt, s_pre, hkv) : nxt;
    const int t0 = cur.ti * TOK;
    if constexpr (F8) {
      Buf8<D> b;
      read_tile8<D, B>(b, &stc[wave][0], tbc, num_blocks, r, gq);
      __builtin_amdgcn_sched_barrier(0);
      tb2 = load_tb<B, TOK>(nxt2, block_tables, max_blocks, s_len);
      load_q<D, F8>(qn, nxt, q, hq, g, r, gq);
      scn = load_scales<B>(tbn, k_scale, v_scale, nxt.j, hkv, num_blocks, gq);
      dma_tile<D, B, F8>(&stn[wave][0], nxt.j, tbn, k_pool, v_pool, hkv, num_blocks, lane);
      const bool full = t0 + TOK <= S && __all(b.ok[0][0] && b.ok[0][1] && b.ok[1][0] && b.ok[1][1]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        f32x4 sco[2];
        qk_tile8<D>(sco, b.k[u], qc);
        const float sk[2] = {scale_log2 * scc.k[u][0], scale_log2 * scc.k[u][1]};
        const float sv[2] = {scc.v[u][0], scc.v[u][1]};
        pv_tile8<D>(st, sco, b.v[u], b.ok[u], t0 + 32 * u, S, full, sk, sv, gq);
      }
    } else {
      Buf<D> b;
      read_tile<D, B>(b, &stc[wave][0], tbc, num_blocks, r, gq);
      // keep the stage's LDS reads ahead of the copies below: an LDS read issued
      // after them would wait for all of them
      __builtin_amdgcn_sched_barrier(0);
      if (k_new != nullptr && has_new_token(packed) && cur.ti == nt_cur - 1) {
        patch_new<D>(b, ntok, pool_tokens(packed) - t0, r, gq);
        // the row's slot, read from wherever the caller keeps it, goes on to the
        // merge kernel (which stores the token): the slot when it is the row's
        // next position, else -1
        if (cur.j == 0 && lane == 0) {
          const int S0 = pool_tokens(packed);
          const bool at_next = next_fits(packed) && ntok.slot >= 0 &&
                               static_cast<int64_t>(ntok.slot) < static_cast<int64_t>(num_blocks) * B &&
                               ntok.slot % B == S0 % B;
          slots_out[cur.n] = at_next ? ntok.slot : -1;
        }
      }
      tb2 = load_tb<B, TOK>(nxt2, block_tables, max_blocks, s_len);
      load_q<D, F8>(qn, nxt, q, hq, g, r, gq);
      if (has_next && wants_new(nxt)) load_new<D>(ntok, nxt, k_new, v_new, slots, hkv, r, gq);
      dma_tile<D, B, F8>(&stn[wave][0], nxt.j, tbn, k_pool, v_pool, hkv, num_blocks, lane);
      const bool full = t0 + 32 <= S && __all(b.blk0 && b.blk1);
      f32x4 sco[2];
      qk_tile<D>(sco, b, qc);
      pv_tile<D>(st, sco, b, t0, S, full, scale_log2, gq);
    }
    const bool seg_end = cur.ti == nt_cur - 1;
    if (seg_end || !has_next) {
      flush<D>(st, cur, piece_start == 0 && seg_end, first_piece ? 0 : 1, wave_id, out, rec, hq, g, r, gq);
      first_piece = false;
      piece_start = 0;
    }
    if (!has_next) return false;
    ++x;
    cur = nxt;
    nxt = nxt2;
    return true;
  };
  while (true) {
    if (!step(std::integral_constant<int, 0>{}, qA, tbA, scA, qB, tbB, scB, tbA)) break;
    if (!step(std::integral_constant<int, 1>{}, qB, tbB, scB, qA, tbA, scA, tbB)) break;
  }
}

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

// The new token of (row n, KV head j) as thread t of the workgroup holds it:
// key chunk t (t < D / 8) and value row d = t (t < D).  Loaded when the merge
// kernel starts, stored when it ends.
template <int D>
struct RowToken {
  int64_t slot;
  uint4 k;
  uint16_t v;
};

template <int D>
__device__ __forceinline__ RowToken<D> load_row_token(const AppendArgs& ap, int n, int j, int hkv) {
  RowToken<D> rt;
  const int64_t src = (static_cast<int64_t>(n) * hkv + j) * D;
  const int t = threadIdx.x;
  rt.slot = ap.slots[n];
  rt.k = t < D / 8 ? *reinterpret_cast<const uint4*>(ap.k_new + src + t * 8) : make_uint4(0, 0, 0, 0);
  rt.v = t < D ? ap.v_new[src + t] : 0;
  return rt;
}

template <int D>
__device__ __forceinline__ void append_row(const AppendArgs& ap, const RowToken<D>& rt, int n, int j, int hkv) {
  if (rt.slot < 0) return;
  const int B = ap.block_size;
  const int64_t pb = rt.slot / B;
  const int off = static_cast<int>(rt.slot % B);
  const int64_t head = pb * hkv + j;
  const int t = threadIdx.x;
  if (t < D / 8) *reinterpret_cast<uint4*>(ap.k_pool + ((head * (D / 8) + t) * B + off) * 8) = rt.k;
  if (t < D) ap.v_pool[(head * D + t) * B + off] = rt.v;
  if (j == 0 && t == 0) {  // the only thread that reads or writes the row
    const int pos = ap.context_lens[n];
    ap.block_tables[static_cast<int64_t>(n) * ap.max_blocks + pos / B] = static_cast<int32_t>(pb);
    ap.context_lens[n] = pos + 1;
  }
}

// Combine the summary records of one segment cut by wave-range boundaries,
// or write zeros for an empty sequence.  Wave h' of the workgroup takes heads
// h', h' + 4, ...; lanes read records in parallel (wave v_lo + lane), so the
// merge costs a few memory latencies rather than one per record.  Records
// combine in wave order, which is tile order.
template <int D>
__device__ __forceinline__ void merge_segment(const float* __restrict__ rec, const int32_t* __restrict__ prefix,
                                              uint16_t* __restrict__ out, int n_seqs, int hq, int hkv, int g,
                                              int64_t total_waves, int j, int n) {
  constexpr int E = D / 64;  // output elements per lane
  const int64_t p_n = prefix[n];
  const int nt = prefix[n + 1] - prefix[n];
  uint16_t* o = out + (static_cast<int64_t>(n) * hq + j * g) * D;
  if (nt == 0) {
    for (int e = threadIdx.x; e < g * D; e += blockDim.x) o[e] = 0;
    return;
  }
  Split sp;
  sp.init(static_cast<int64_t>(hkv) * prefix[n_seqs], total_waves);
  const int64_t a = hkv * p_n + static_cast<int64_t>(j) * nt;  // first tile of the segment
  const int64_t b = a + nt;                                    // one past its last tile
  const int64_t v_lo = sp.wave_of(a);
  const int64_t v_hi = sp.wave_of(b - 1);
  if (v_lo == v_hi) return;  // finished inside one wave
  const bool lo_second = a > sp.start(v_lo);  // the segment is not the first piece of wave v_lo
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // the record of wave v for head h, or nullptr for a wave with an empty range
  auto record = [&](int64_t v, int h) -> const float* {
    if (v > v_hi || sp.start(v) == sp.start(v + 1)) return nullptr;
    const int slot = (v == v_lo && lo_second) ? 1 : 0;
    return rec + ((v * 2 + slot) * g + h) * (D + 4);
  };
  if (v_hi - v_lo < 8) {
    // up to 8 pieces (the usual case): the maxima, sums and value rows of all
    // pieces load together, in one memory round trip
    const int cnt = static_cast<int>(v_hi - v_lo + 1);
    for (int h = wave; h < g; h += 4) {
      const float* mine = lane < cnt ? record(v_lo + lane, h) : nullptr;
      const float* ml = mine ? mine : rec;  // any valid address; unused
      const float m_l = ml[0], z_l = ml[1];
      float val[8][E];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float* rk = k < cnt ? record(v_lo + k, h) : nullptr;
        rk = rk ? rk : rec;  // weighted by zero below
#pragma unroll
        for (int e = 0; e < E; ++e) val[k][e] = rk[4 + lane + 64 * e];
      }
      float mx = mine ? m_l : -INFINITY;
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
      const float f = mine ? __builtin_amdgcn_exp2f(m_l - mx) : 0.f;
      float zz = mine ? f * z_l : 0.f;
#pragma unroll
      for (int sh = 32; sh >= 1; sh >>= 1) zz += __shfl_xor(zz, sh);
      float uu[E];
#pragma unroll
      for (int e = 0; e < E; ++e) uu[e] = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float fk = __shfl(f, k);  // zero for k >= cnt and empty ranges
#pragma unroll
        for (int e = 0; e < E; ++e) uu[e] += fk * val[k][e];
      }
      const float inv = 1.f / zz;
#pragma unroll
      for (int e = 0; e < E; ++e) o[h * D + lane + 64 * e] = f32_to_bf16_bits(uu[e] * inv);
    }
    return;
  }
  for (int h = wave; h < g; h += 4) {
    float mx = -INFINITY;
    for (int64_t base = v_lo; base <= v_hi; base += 64) {
      const float* rr = record(base + lane, h);
      if (rr) mx = fmaxf(mx, rr[0]);
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) mx = fmaxf(mx, __shfl_xor(mx, sh));
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
          fk[i] = __shfl(f, k & 63);
          if (!rk) fk[i] = 0.f;
          rk = rk ? rk : rec;  // any valid address; weighted by zero
#pragma unroll
          for (int e = 0; e < E; ++e) val[i][e] = rk[4 + lane + 64 * e];
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
          for (int e = 0; e < E; ++e) uu[e] += fk[i] * val[i][e];
      }
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) zz += __shfl_xor(zz, sh);
    const float inv = 1.f / zz;
#pragma unroll
    for (int e = 0; e < E; ++e) o[h * D + lane + 64 * e] = f32_to_bf16_bits(uu[e] * inv);
  }
}

// Second kernel of a decode: one workgroup per (KV head, sequence) merges the
// segment's pieces; for pa_decode_step it also stores the new token and moves
// the row forward.
template <int D>
__global__ __launch_bounds__(256) void merge_stream(const float* __restrict__ rec,
                                                    const int32_t* __restrict__ prefix, uint16_t* __restrict__ out,
                                                    int n_seqs, int hq, int hkv, int g, int64_t total_waves,
                                                    AppendArgs ap) {
  const int j = blockIdx.x;
  const int n = blockIdx.y;
  if (ap.k_new == nullptr) {
    merge_segment<D>(rec, prefix, out, n_seqs, hq, hkv, g, total_waves, j, n);
    return;
  }
  const RowToken<D> rt = load_row_token<D>(ap, n, j, hkv);  // in flight during the merge
  merge_segment<D>(rec, prefix, out, n_seqs, hq, hkv, g, total_waves, j, n);
  append_row<D>(ap, rt, n, j, hkv);
}

template <int D, int B>
const void* stream_kernel() {
  return reinterpret_cast<const void*>(&decode_stream<D, B, false>);
}

const void* stream_kernel_for(int d, int b) {
  if (d == 128) return b == 8 ? stream_kernel<128, 8>() : (b == 16 ? stream_kernel<128, 16>() : stream_kernel<128, 32>());
  return b == 8 ? stream_kernel<64, 8>() : (b == 16 ? stream_kernel<64, 16>() : stream_kernel<64, 32>());
}

size_t stream_lds(int n_seqs) { return (2 * static_cast<size_t>(n_seqs) + 1) * sizeof(int32_t); }

// Resident workgroups per CU and CU count of the current device, cached.
// Without a device (host-only use) the MI355X figures (256 CUs) and 2
// workgroups per CU are assumed.
struct DeviceShape {
  int cus = 256;
  int wg_per_cu[2][3] = {{2, 2, 2}, {2, 2, 2}};
};

const DeviceShape& device_shape() {
  static DeviceShape shapes[16];
  static bool ready[16] = {};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
    (void)hipGetLastError();
    static DeviceShape fallback;
    return fallback;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ready[dev]) {
    DeviceShape s;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0) s.cus = cus;
    const int ds[2] = {64, 128}, bs[3] = {8, 16, 32};
    for (int a = 0; a < 2; ++a)
      for (int c = 0; c < 3; ++c) {
        int nb = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, stream_kernel_for(ds[a], bs[c]), 256,
                                                         stream_lds(kMaxSeqs)) == hipSuccess &&
            nb > 0)
          s.wg_per_cu[a][c] = nb;
      }
    (void)hipGetLastError();
    shapes[dev] = s;
    ready[dev] = true;
  }
  return shapes[dev];
}

}  // namespace

bool stream_eligible(int num_seqs, int g, int d, int block_size, int dtype) {
  return dtype == PA_BF16 && (d == 64 || d == 128) && g >= 1 && g <= 16 &&
         (block_size == 8 || block_size == 16 || block_size == 32) && num_seqs <= kMaxSeqs;
}

bool stream_eligible_fp8(int num_seqs, int g, int d, int block_size) {
  return stream_eligible(num_seqs, g, d, block_size, PA_BF16);
}

StreamPlan stream_plan(int num_seqs, int hq, int hkv, int d, int block_size, int max_ctx, bool fp8) {
  const DeviceShape& ds = device_shape();
  const int ai = d == 128 ? 1 : 0;
  const int bi = block_size == 8 ? 0 : (block_size == 16 ? 1 : 2);
  StreamPlan p;
  // One workgroup (4 waves, one per SIMD) per CU: with two or more per CU the
  // oldest waves win the memory pipe and the split's completion times spread.
  int per_cu = 1;
  if (const char* env = std::getenv("PA_STREAM_WG_PER_CU")) {  // tuning sweeps
    const int v = std::atoi(env);
    if (v >= 1 && v <= ds.wg_per_cu[ai][bi]) per_cu = v;
  }
  int64_t wgs = static_cast<int64_t>(ds.cus) * per_cu;
  // no more waves than tiles / 2 (upper bound of the work from max_context_len)
  const int tok = fp8 ? kTok<true> : kTok<false>;
  const int64_t t_bound = static_cast<int64_t>(num_seqs) * hkv * ((max_ctx + tok - 1) / tok);
  const int64_t by_work = (t_bound + 2 * kSW - 1) / (2 * kSW);
  if (by_work < wgs) wgs = by_work;
  if (wgs < 1) wgs = 1;
  p.workgroups = static_cast<int>(wgs);
  const int g = hq / hkv;
  const int64_t waves = wgs * kSW;
  p.prefix_offset = 0;
  const size_t prefix_bytes = ((static_cast<size_t>(num_seqs) + 1) * sizeof(int32_t) + 255) / 256 * 256;
  p.slots_offset = p.prefix_offset + prefix_bytes;
  p.records_offset = p.slots_offset + prefix_bytes;
  p.workspace_bytes = p.records_offset + static_cast<size_t>(waves) * 2 * g * (d + 4) * sizeof(float);
  p.lds_bytes = stream_lds(num_seqs);
  return p;
}

template <int D, int B, bool F8>
static void launch_stream_db(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v,
                             const int32_t* bt, const int32_t* cl, void* out, void* ws, int n, int hq, int hkv,
                             int max_blocks, int num_blocks, float scale_log2, const StepInputs* step,
                             const float* k_scale, const float* v_scale) {
  char* base = static_cast<char*>(ws);
  int32_t* prefix = reinterpret_cast<int32_t*>(base + p.prefix_offset);
  int32_t* slots_ws = reinterpret_cast<int32_t*>(base + p.slots_offset);
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
    ap.slots = slots_ws;  // the decode kernel copies each row's slot there
    ap.block_tables = const_cast<int32_t*>(bt);
    ap.context_lens = const_cast<int32_t*>(cl);
    ap.max_blocks = max_blocks;
    ap.block_size = B;
  }
  decode_stream<D, B, F8><<<dim3(p.workgroups), dim3(256), p.lds_bytes, s>>>(
      static_cast<const uint16_t*>(q), k, v, bt, cl, static_cast<uint16_t*>(out), rec, prefix, n, hq, hkv, g,
      max_blocks, num_blocks, scale_log2, ap.k_new, ap.v_new, slots_in, slots_ws, k_scale, v_scale);
  merge_stream<D><<<dim3(hkv, n), dim3(256), 0, s>>>(rec, prefix, static_cast<uint16_t*>(out), n, hq, hkv, g,
                                                     static_cast<int64_t>(p.workgroups) * kSW, ap);
}

int launch_stream(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v, const int32_t* bt,
                  const int32_t* cl, void* out, void* ws, int n, int hq, int hkv, int d, int block_size,
                  int max_blocks, int num_blocks, float scale_log2, const StepInputs* step, const float* k_scale,
                  const float* v_scale) {
  const bool f8 = k_scale != nullptr;
  if (f8 && step) return PA_ERR_UNSUPPORTED;
#define PA_STREAM_CASE(DD, BB)                                                                               \
  if (d == DD && block_size == BB) {                                                                         \
    if (f8)                                                                                                  \
      launch_stream_db<DD, BB, true>(p, s, q, k, v, bt, cl, out, ws, n, hq, hkv, max_blocks, num_blocks,     \
                                     scale_log2, nullptr, k_scale, v_scale);                                 \
    else                                                                                                     \
      launch_stream_db<DD, BB, false>(p, s, q, k, v, bt, cl, out, ws, n, hq, hkv, max_blocks, num_blocks,    \
                                      scale_log2, step, nullptr, nullptr);                                   \
    return launch_status();                                                                                  \
  }
  PA_STREAM_CASE(128, 16)
  PA_STREAM_CASE(128, 8)
  PA_STREAM_CASE(128, 32)
  PA_STREAM_CASE(64, 16)
  PA_STREAM_CASE(64, 8)
  PA_STREAM_CASE(64, 32)
#undef PA_STREAM_CASE
  return PA_ERR_UNSUPPORTED;
}

}  // namespace pa

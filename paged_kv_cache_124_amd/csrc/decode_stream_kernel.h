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
// Per tile the matrix-core roles of decode_tile.h, with the G query heads of
// the KV head as the 16 columns (head r, padding for r >= G).
//
// Pool layout (per layer): K and V [num_blocks][Hkv][B][D] (rows of D bf16
// values or D one-byte codes).


#pragma once

#include <type_traits>

#include "codes.h"
#include "common.h"
#include "decode_stream.h"
#include "decode_tile.h"

namespace pa {
namespace {

constexpr int kMaxSeqs = 3072;  // lengths and tile prefix sums live in LDS beside the stages

// ---- caches of one-byte codes (FP8 E4M3 or INT8) --------------------------------
//
// A stored code c stands for value(c) * scale, one fp32 scale per (block, KV
// head) for keys and one for values.  Both products run as fp16 MFMAs on the
// codes' values; the scales are applied outside them: the key scale
// multiplies a token's score, the value scale its probability in P.V (the
// weight sum uses the unscaled probability).
//   FP8: gfx950 converts two E4M3 codes to two fp16 values in one
//   instruction, exactly (every E4M3 value is an fp16 value).
//   INT8: the fp16 number with high byte 0x64 and low byte c ^ 0x80 is
//   1024 + (c + 128), exactly.  One byte permute builds two of them from a
//   word of four codes and one XOR per word flips the four sign bits: 0.75
//   instructions per code.  The common offset kI8Offset = 1152 comes out
//   afterwards: from a score as 1152 times the sum of the head's fp16 query,
//   from P.V as 1152 times the sum of the tile's P column, on the tile's own
//   accumulator (so the offset never grows with the context).
//   Q: each head's row is scaled by the power of two that puts its largest
//   magnitude in [2^14, 2^15) before the fp16 conversion (exact for every
//   bf16 value down to 2^-28 of that magnitude); the score takes the power
//   back.
//   P: with fp16's 11 significant bits one MFMA per product suffices.  Its
//   range is kept by weighing p * (value scale / vref), vref the largest
//   value scale of the segment so far -- raised tile by tile like the running
//   maximum, the accumulator rescaled with it -- and the segment's output is
//   multiplied by vref when it is written.
// A 64-token tile is two 32-token sub-tiles under one online-softmax update.

// Register image of a staged tile of codes for lane (r, gq).
template <int D>
struct Buf8 {
  uint4 k[2][2][D / 64];     // [sub-tile][slab] key row 16 slab + r: the 16-byte chunks of d quarter gq
  uint32_t v[2][2][D / 16];  // [sub-tile][slab][mm] tokens 4 gq .. 4 gq + 3 of the slab at d = 16 mm + r
  bool ok[2][2];             // the block of that value group is in the pool
};

// Scales of the blocks of the lane's token groups (0 where the block is missing),
// from the interleaved array [num_blocks][Hkv][2] (key, value).
struct Sc8 {
  float k[2][2], v[2][2];  // [sub-tile][slab]
};

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The fp16 image of INT8 code c is c + kI8Offset.
constexpr float kI8Offset = 1152.f;

// Eight codes (two words, lowest byte first) as eight fp16 values: the E4M3
// values, or the INT8 codes plus kI8Offset.
template <bool I8>
__device__ __forceinline__ f16x8 codes8_to_f16(uint32_t lo, uint32_t hi) {
  if constexpr (I8) {
    const uint32_t a = lo ^ 0x80808080u, b = hi ^ 0x80808080u;
    // selector bytes 0-3 take bytes of the flipped code word, 4 the byte 0x64
    return __builtin_bit_cast(f16x8, uint4{__builtin_amdgcn_perm(0x64646464u, a, 0x04010400u),
                                           __builtin_amdgcn_perm(0x64646464u, a, 0x04030402u),
                                           __builtin_amdgcn_perm(0x64646464u, b, 0x04010400u),
                                           __builtin_amdgcn_perm(0x64646464u, b, 0x04030402u)});
  } else {
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
}

// Query operand of a tile of codes: lane (r, gq) holds head r's elements
// d = gq D / 4 + 8 jj .. + 7 (the key chunks the lane holds), scaled by 2^k.
template <int D>
struct QOp16 {
  f16x8 q[D / 32];
  float unscale;  // 2^-k
  float offset;   // INT8: kI8Offset times the sum of head r's fp16 elements
};

template <int D, bool I8>
__device__ __forceinline__ void load_q16(QOp16<D>& qo, TilePos t, const uint16_t* __restrict__ q, int hq, int g,
                                         int r, int gq) {
  // padding columns r >= G read head 0 of the group; their results are never used
  const uint16_t* qh = q + (static_cast<int64_t>(t.n) * hq + t.j * g + (r < g ? r : 0)) * D;
  uint4 raw[D / 32];
  float amax = 0.f;
#pragma unroll
  for (int jj = 0; jj < D / 32; ++jj) {
    raw[jj] = *reinterpret_cast<const uint4*>(qh + gq * (D / 4) + 8 * jj);
    const uint32_t w[4] = {raw[jj].x, raw[jj].y, raw[jj].z, raw[jj].w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[e] << 16)), fabsf(__uint_as_float(w[e] & 0xffff0000u))));
  }
  amax = max_across_groups(amax);
  int ex = 0;
  if (amax > 0.f && amax <= __FLT_MAX__) frexpf(amax, &ex);  // amax in [2^(ex-1), 2^ex)
  const int k = min(max(15 - ex, -126), 126);
  const float up = ldexpf(1.f, k);
  qo.unscale = ldexpf(1.f, -k);
  float sum = 0.f;
#pragma unroll
  for (int jj = 0; jj < D / 32; ++jj) {
    const uint32_t w[4] = {raw[jj].x, raw[jj].y, raw[jj].z, raw[jj].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const _Float16 lo = static_cast<_Float16>(__uint_as_float(w[e] << 16) * up);
      const _Float16 hi = static_cast<_Float16>(__uint_as_float(w[e] & 0xffff0000u) * up);
      qo.q[jj][2 * e] = lo;
      qo.q[jj][2 * e + 1] = hi;
      sum += static_cast<float>(lo) + static_cast<float>(hi);
    }
  }
  if constexpr (I8) {
    sum = sum_across_groups(sum);
    qo.offset = kI8Offset * sum;
  } else {
    qo.offset = 0.f;
  }
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
__device__ __forceinline__ Sc8 load_scales(const Tb<64 / B>& tb, const float* __restrict__ scales, int j, int hkv,
                                           int num_blocks, int gq) {
  Sc8 sc;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int e = group_block<B>(tb, 32 * u + 16 * a, gq);
      const bool ok = e >= 0 && e < num_blocks;
      const int64_t idx = static_cast<int64_t>(ok ? e : 0) * hkv + j;
      const float2 kv = *reinterpret_cast<const float2*>(scales + 2 * idx);  // one 8-byte load per (block, head)
      sc.k[u][a] = ok ? kv.x : 0.f;
      sc.v[u][a] = ok ? kv.y : 0.f;
    }
  return sc;
}

// Operands of a staged tile of codes (rows of D bytes, chunks swizzled as in
// dma_tile).  Key: row 32 u + 16 a + r, the chunks of d quarter gq.  Value:
// one transposing read per (sub-tile u, d block mm) gives the lane the codes
// of tokens 4 gq .. + 3 of both slabs at d = 16 mm + r: in-lane i = 2 j + h of
// the 16-lane group points at d = 16 mm + 8 h .. + 7 of token 4 gq + j (j < 4,
// slab 0) or 16 + 4 gq + j - 4 (slab 1).
template <int D, int B>
__device__ __forceinline__ void read_tile8(Buf8<D>& b, const unsigned char* stage, const Tb<64 / B>& tb, int num_blocks,
                                           int r, int gq) {
  constexpr int RB = D;
  const int vj = r >> 1, vh = r & 1;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int tk = 32 * u + 16 * a + r;  // key row
      const int sk = stage_swz<D, true>(tk);
#pragma unroll
      for (int w = 0; w < D / 64; ++w)
        b.k[u][a][w] = *reinterpret_cast<const uint4*>(stage + tk * RB + (((gq * (D / 64) + w) ^ sk) << 4));
      const int e = group_block<B>(tb, 32 * u + 16 * a, gq);
      b.ok[u][a] = e >= 0 && e < num_blocks;
    }
    const int tv = 32 * u + (vj < 4 ? 4 * gq + vj : 16 + 4 * gq + vj - 4);  // the value row this lane points at
    const int sv = stage_swz<D, true>(tv);
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm) {
      const uint2 v = lds_read_tr8(stage + kStageHalf<D> + tv * RB + ((mm ^ sv) << 4) + vh * 8);
      b.v[u][0][mm] = v.x;
      b.v[u][1][mm] = v.y;
    }
  }
}

// One staged 64-token tile of codes into the lane's running state: scores of
// both sub-tiles, one online-softmax update, P.V.  sc holds the tile's key and
// value scales.  FULL: all 64 tokens present (the usual tile), so no score is
// masked and no code zeroed; a separate instance takes the partial tiles.
template <int D, bool I8, bool FULL>
__device__ __forceinline__ void codes_tile(Acc<D>& st, const Buf8<D>& b, const Sc8& sc, const QOp16<D>& qc, int t0,
                                           int S, float scale_log2, int gq) {
  // scores: [sub-tile u][slab a][i] is token 32 u + 16 a + 4 gq + i for head r
  f32x4 s[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      s[u][a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < D / 32; ++jj) {
        const uint4 c = b.k[u][a][jj >> 1];
        const f16x8 kop = (jj & 1) ? codes8_to_f16<I8>(c.z, c.w) : codes8_to_f16<I8>(c.x, c.y);
        s[u][a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qc.q[jj], s[u][a], 0, 0, 0);
      }
    }
  int n[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int a = 0; a < 2; ++a)
      n[u][a] = FULL ? 4 : (b.ok[u][a] ? min(max(S - (t0 + 32 * u + 16 * a + 4 * gq), 0), 4) : 0);
  float x[2][2][4];
  float tmax = -INFINITY;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float sk = scale_log2 * sc.k[u][a] * qc.unscale;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[u][a][i] = i < n[u][a] ? (s[u][a][i] - qc.offset) * sk : -INFINITY;
        tmax = fmaxf(tmax, x[u][a][i]);
      }
    }
  tmax = max_across_groups(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;
  // the value-scale reference: the largest scale of the segment so far (wave-uniform)
  float tv = fmaxf(fmaxf(sc.v[0][0], sc.v[0][1]), fmaxf(sc.v[1][0], sc.v[1][1]));
  tv = max_across_groups(tv);
  float f = alpha;  // rescale of the accumulated P.V
  if (tv > st.vref) {
    f *= st.vref / tv;
    st.vref = tv;
  }
  const float inv = st.vref > 0.f ? 1.f / st.vref : 0.f;
  float psum = 0.f, pcol = 0.f;
  f16x8 P[2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const float w = sc.v[u][a] * inv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[u][a][i] - m_new);
        psum += p;
        const _Float16 h = static_cast<_Float16>(p * w);
        P[u][4 * a + i] = h;
        pcol += static_cast<float>(h);
      }
    }
  st.z = st.z * alpha + psum;
  if constexpr (I8) {
    // every code is finite, and a missing token has P = 0: no masking
    pcol = sum_across_groups(pcol);
    // the tile's products start from minus the offset, so they come out without it
    const float noff = -kI8Offset * pcol;
    const f32x4 t0v{noff, noff, noff, noff};
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm) {
      f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8_to_f16<true>(b.v[0][0][mm], b.v[0][1][mm]), P[0], t0v,
                                                       0, 0, 0);
      t = __builtin_amdgcn_mfma_f32_16x16x32_f16(codes8_to_f16<true>(b.v[1][0][mm], b.v[1][1][mm]), P[1], t, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) st.o[mm][i] = st.o[mm][i] * f + t[i];
    }
  } else {
    if (__any(f != 1.f)) {
#pragma unroll
      for (int mm = 0; mm < D / 16; ++mm) st.o[mm] *= f;
    }
    // zero the codes of missing tokens: stale or NaN codes must not reach P.V (code 0 is 0)
    uint32_t msk[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int a = 0; a < 2; ++a) msk[u][a] = FULL || n[u][a] >= 4 ? 0xffffffffu : (1u << (8 * n[u][a])) - 1u;
#pragma unroll
    for (int mm = 0; mm < D / 16; ++mm)
#pragma unroll
      for (int u = 0; u < 2; ++u)
        st.o[mm] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
            codes8_to_f16<false>(b.v[u][0][mm] & msk[u][0], b.v[u][1][mm] & msk[u][1]), P[u], st.o[mm], 0, 0, 0);
  }
}

// End of a piece of segment t: write the normalised output (whole segment) or a summary record.
// The accumulated P.V is omul times the true one's (1, or a cache of codes' vref).
// With whole_rec non-null (a decode step over a cache of codes, whose merge
// kernel adds the new token) a whole segment leaves its summary in
// whole_rec[n][j] instead of its output.
template <int D>
__device__ __forceinline__ void flush(Acc<D>& st, TilePos t, bool whole, int slot, int64_t wave_id, uint16_t* out,
                                      float* rec, float* whole_rec, int hq, int hkv, int g, int r, int gq,
                                      float omul) {
  const float zt = sum_across_groups(st.z);
  if (r < g) {
    if (whole && whole_rec == nullptr) {
      const float inv = zt > 0.f ? omul / zt : 0.f;  // every token left out: zeros
      uint16_t* o = out + (static_cast<int64_t>(t.n) * hq + t.j * g + r) * D + 4 * gq;
#pragma unroll
      for (int mm = 0; mm < D / 16; ++mm) {
        const uint32_t lo = f32_to_bf16_bits(st.o[mm][0] * inv) | (uint32_t(f32_to_bf16_bits(st.o[mm][1] * inv)) << 16);
        const uint32_t hi = f32_to_bf16_bits(st.o[mm][2] * inv) | (uint32_t(f32_to_bf16_bits(st.o[mm][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(o + 16 * mm) = make_uint2(lo, hi);
      }
    } else {
      float* rr = whole ? whole_rec + ((static_cast<int64_t>(t.n) * hkv + t.j) * g + r) * (D + 4)
                        : rec + (static_cast<int64_t>(wave_id * 2 + slot) * g + r) * (D + 4);
#pragma unroll
      for (int mm = 0; mm < D / 16; ++mm) *reinterpret_cast<f32x4*>(rr + 4 + 16 * mm + 4 * gq) = st.o[mm] * omul;
      if (gq == 0) {
        rr[0] = st.m;
        rr[1] = zt;
      }
    }
  }
  reset(st);
}


// What a step needs to know about one tile of the list: its (row, KV head,
// tile), the row's packed tokens and the segment's tile count.  Each lane
// works out one tile of a window of 64 consecutive tiles of the wave's range
// from the tables in LDS (a binary search over the prefix sums); a step reads
// the tile after next from its lane (readlane, wave-uniform results), so no LDS
// lookup lies between one tile's copies and the next's.  A new window is built
// once per 62 tiles.
struct STile {
  int n, j, ti, packed, nt;
};

__device__ __forceinline__ STile stile_of(int64_t x, const int32_t* s_pre, const int32_t* s_len, int n_seqs,
                                          int hkv) {
  int lo = 0, hi = n_seqs - 1;  // last n with hkv * s_pre[n] <= x (a row with tiles)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (static_cast<int64_t>(hkv) * s_pre[mid] <= x) lo = mid; else hi = mid - 1;
  }
  STile t;
  t.n = lo;
  t.nt = tiles_of(s_pre, lo);
  const int64_t rem = x - static_cast<int64_t>(hkv) * s_pre[lo];
  t.j = static_cast<int>(rem / t.nt);
  t.ti = static_cast<int>(rem - static_cast<int64_t>(t.j) * t.nt);
  t.packed = s_len[lo];
  return t;
}

__device__ __forceinline__ STile lane_stile(const STile& d, int idx) {
  STile t;
  t.n = __builtin_amdgcn_readlane(d.n, idx);
  t.j = __builtin_amdgcn_readlane(d.j, idx);
  t.ti = __builtin_amdgcn_readlane(d.ti, idx);
  t.packed = __builtin_amdgcn_readlane(d.packed, idx);
  t.nt = __builtin_amdgcn_readlane(d.nt, idx);
  return t;
}

__device__ __forceinline__ TilePos pos_of(const STile& t) { return TilePos{t.n, t.j, t.ti}; }

// Table entries of a tile's blocks.  Always loaded (index clamped into the
// row) and replaced by -1 past the end of the row's tokens in the pool, so no
// load sits behind a branch and the compiler keeps the pipeline's loads in flight.
template <int B, int TOK>
__device__ __forceinline__ Tb<TOK / B> load_tb_s(const STile& t, const int32_t* __restrict__ block_tables,
                                                 int max_blocks) {
  const int32_t* row = block_tables + static_cast<int64_t>(t.n) * max_blocks;
  const int S = pool_tokens(t.packed);
  const int t0 = t.ti * TOK;
  Tb<TOK / B> tb;
#pragma unroll
  for (int i = 0; i < TOK / B; ++i) {
    const int e = row[min(t0 / B + i, max_blocks - 1)];
    tb.blk[i] = t0 + i * B < S ? e : -1;
  }
  return tb;
}

template <int D, int B, int KV>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1))) void decode_stream(
    const uint16_t* __restrict__ q, const void* __restrict__ k_pool, const void* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    float* __restrict__ rec, int32_t* __restrict__ prefix_out, int n_seqs, int hq, int hkv, int g, int max_blocks,
    int num_blocks, float scale_log2, const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const int32_t* __restrict__ slots, int32_t* __restrict__ slots_out, const float* __restrict__ scales,
    float* __restrict__ whole_rec, int32_t* __restrict__ lens_out) {
  constexpr bool F8 = KV != kKvBf16;  // one-byte codes (E4M3 or INT8) with scales
  constexpr bool I8 = KV == kKvInt8;
  constexpr int TOK = kTok<F8>;
  constexpr int NB = TOK / B;
  extern __shared__ int32_t sm[];
  int32_t* s_len = sm;            // [n_seqs] packed attended-token counts (pool part clamped to the table)
  int32_t* s_pre = sm + n_seqs;   // [n_seqs + 1] tile prefix sums
  __shared__ int32_t s_wsum[kSW];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: stage addresses go to m0 from scalars
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
  if (blockIdx.x == 0) {
    for (int i = tid; i <= n_seqs; i += 256) prefix_out[i] = s_pre[i];
    if (lens_out != nullptr)  // the rows as this decode saw them, for a merge kernel that moves them on
      for (int i = tid; i < n_seqs; i += 256) lens_out[i] = s_len[i];
  }
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

  // the window of tiles xb .. xb + 63 (past the range: its last tile again)
  int64_t xb = x0;
  STile mine = stile_of(min(xb + lane, x1 - 1), s_pre, s_len, n_seqs, hkv);
  STile cur = lane_stile(mine, 0);
  int piece_start = cur.ti;  // first tile of the current piece
  bool first_piece = true;

  Acc<D> st;
  reset(st);
  // Two LDS stages per wave: while tile x is computed (from registers read
  // out of one stage), tile x + 1's keys and values stream into the other
  // stage and the table entries of tile x + 2 load as well.  The table-entry
  // loads are unconditional (a missing successor repeats the current tile's
  // addresses); a wave's last tile issues no copy.
  // The queries are those of the segment: loaded when a segment starts, not
  // again for each of its tiles.
  std::conditional_t<F8, QOp16<D>, QOp<D>> qc;
  auto segment_queries = [&](const STile& t) {
    if constexpr (F8)
      load_q16<D, I8>(qc, pos_of(t), q, hq, g, r, gq);
    else
      load_q<D, false>(qc, pos_of(t), q, hq, g, r, gq);
  };
  STile nxt = lane_stile(mine, 1);  // the range's only tile again when it has one
  Tb<NB> tbA = load_tb_s<B, TOK>(cur, block_tables, max_blocks);
  Tb<NB> tbB = load_tb_s<B, TOK>(nxt, block_tables, max_blocks);
  segment_queries(cur);
  dma_tile<D, B, F8>(&g_stage0[wave][0], cur.j, tbA, k_pool, v_pool, hkv, num_blocks, lane);
  // FP8: the scales of a tile's blocks travel with it, one tile ahead like its Q
  Sc8 scA{}, scB{};
  if constexpr (F8) scA = load_scales<B>(tbA, scales, cur.j, hkv, num_blocks, gq);

  int64_t x = x0;
  // One step: tile `cur` (staged in stage SC, blocks tbc) is computed while
  // `nxt` streams into the other stage (its blocks tbn are known) and the
  // table entries of the tile after it load into tb2.  Returns false after
  // the last tile.
  // the step's new token, for tiles that end a segment holding one
  auto wants_new = [&](const STile& t) -> bool {
    return !F8 && k_new != nullptr && has_new_token(t.packed) && t.ti == t.nt - 1;
  };
  // one buffer: a step patches its tile before it loads the next tile's token
  NewTok<D> ntok;
  // A store issued between two tiles makes the next stage wait for it as well
  // (loads and stores count in one in-order counter).  So in the bf16 kernel
  // the wave's first summary or output written before its last tile, and its
  // first forwarded slot, are held here and stored after the last tile.  (The
  // kernels over codes keep storing at once: holding the state there cost more
  // in registers than the wait: FP8 +0.6 us, INT8 +2.5 us per step.)
  Acc<D> pend;
  reset(pend);
  TilePos pend_pos{0, 0, 0};
  bool pend_whole = false, has_pend = false;
  int pend_slot = 0;
  int pend_row = -1, pend_row_slot = -1;  // forwarded slot: row, value (lane 0)
  auto forward_slot = [&](int n, int v) {
    if (!F8 && pend_row < 0) {
      pend_row = n;
      pend_row_slot = v;
    } else {
      slots_out[n] = v;
    }
  };
  if (wants_new(cur)) load_new<D>(ntok, pos_of(cur), k_new, v_new, slots, hkv, r, gq);
  auto step = [&](auto sc_tag, const Tb<NB>& tbc, const Sc8& scc, const Tb<NB>& tbn, Sc8& scn,
                  Tb<NB>& tb2) -> bool {
    constexpr int SC = decltype(sc_tag)::value;
    unsigned char(&stc)[4][kStageBytes] = SC == 0 ? g_stage0 : g_stage1;
    unsigned char(&stn)[4][kStageBytes] = SC == 0 ? g_stage1 : g_stage0;
    // The compiler orders any LDS read after every outstanding LDS copy, so the
    // current stage is read into registers first; the next tile's copies are
    // issued after it and stay in flight through this tile's compute.
    const bool has_next = x + 1 < x1;
    const int packed = cur.packed;
    const int S = attended_tokens(packed);
    const int nt_cur = cur.nt;
    // the tile after next, from the window (rebuilt when used up)
    const int64_t x2 = min(x + 2, x1 - 1);
    if (x2 - xb >= 64) {
      xb = x2;
      mine = stile_of(min(xb + lane, x1 - 1), s_pre, s_len, n_seqs, hkv);
    }
    const STile nxt2 = lane_stile(mine, static_cast<int>(x2 - xb));
    const int t0 = cur.ti * TOK;
    if constexpr (F8) {
      Buf8<D> b;
      wait_stage_copies();
      read_tile8<D, B>(b, &stc[wave][0], tbc, num_blocks, r, gq);
      __builtin_amdgcn_sched_barrier(0);
      // a step over codes: the row's slot, read where the row's head-0 segment
      // ends and handed to the merge kernel through slots_out (read early, stored
      // after this tile's compute)
      const bool row_end = whole_rec != nullptr && cur.j == 0 && cur.ti == nt_cur - 1;
      int row_slot = -1;
      if (row_end) row_slot = slots[cur.n];
      tb2 = load_tb_s<B, TOK>(nxt2, block_tables, max_blocks);
      scn = load_scales<B>(tbn, scales, nxt.j, hkv, num_blocks, gq);
      if (has_next) dma_tile<D, B, F8>(&stn[wave][0], nxt.j, tbn, k_pool, v_pool, hkv, num_blocks, lane);
      const bool full = t0 + TOK <= S && __all(b.ok[0][0] && b.ok[0][1] && b.ok[1][0] && b.ok[1][1]);
      if (full)
        codes_tile<D, I8, true>(st, b, scc, qc, t0, S, scale_log2, gq);
      else
        codes_tile<D, I8, false>(st, b, scc, qc, t0, S, scale_log2, gq);
      if (row_end && lane == 0) forward_slot(cur.n, row_slot);
    } else {
      Buf<D> b;
      wait_stage_copies();
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
          forward_slot(cur.n, at_next ? ntok.slot : -1);
        }
      }
      tb2 = load_tb_s<B, TOK>(nxt2, block_tables, max_blocks);
      if (has_next && wants_new(nxt)) load_new<D>(ntok, pos_of(nxt), k_new, v_new, slots, hkv, r, gq);
      if (has_next) dma_tile<D, B, F8>(&stn[wave][0], nxt.j, tbn, k_pool, v_pool, hkv, num_blocks, lane);
      const bool full = t0 + 32 <= S && __all(b.blk0 && b.blk1);
      f32x4 sco[2];
      qk_tile<D>(sco, b, qc);
      // at a segment's last tile the next segment's queries load here, while
      // the tile's softmax and P.V run: qc is free once the score products
      // have read it (issued after the tile's math, they held up the next wait)
      if (has_next && cur.ti == nt_cur - 1) segment_queries(nxt);
      // constant flags, so that the full tile (the usual one) carries no masking
      if (full)
        pv_tile<D>(st, sco, b, t0, S, true, scale_log2, gq);
      else
        pv_tile<D>(st, sco, b, t0, S, false, scale_log2, gq);
    }
    const bool seg_end = cur.ti == nt_cur - 1;
    if (seg_end || !has_next) {
      const bool whole = piece_start == 0 && seg_end;
      const int slot = first_piece ? 0 : 1;
      if (!F8 && has_next && !has_pend) {
        pend = st;
        pend_pos = pos_of(cur);
        pend_whole = whole;
        pend_slot = slot;
        has_pend = true;
        reset(st);
      } else {
        flush<D>(st, pos_of(cur), whole, slot, wave_id, out, rec, whole_rec, hq, hkv, g, r, gq, F8 ? st.vref : 1.f);
      }
      first_piece = false;
      piece_start = 0;
    }
    if (!has_next) {
      if constexpr (!F8) {
        if (has_pend) flush<D>(pend, pend_pos, pend_whole, pend_slot, wave_id, out, rec, whole_rec, hq, hkv, g, r, gq, 1.f);
        if (lane == 0 && pend_row >= 0) slots_out[pend_row] = pend_row_slot;
      }
      return false;
    }
    if (F8 && seg_end) segment_queries(nxt);  // the bf16 tile loaded them after its score products
    ++x;
    cur = nxt;
    nxt = nxt2;
    return true;
  };
  while (true) {
    if (!step(std::integral_constant<int, 0>{}, tbA, scA, tbB, scB, tbA)) break;
    if (!step(std::integral_constant<int, 1>{}, tbB, scB, tbA, scA, tbB)) break;
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
    merge_segment<D>(rec, prefix, out, n_seqs, hq, hkv, g, g, total_waves, j, n);
    return;
  }
  const RowToken<D> rt = load_row_token<D>(ap, n, j, hkv);  // in flight during the merge
  merge_segment<D>(rec, prefix, out, n_seqs, hq, hkv, g, g, total_waves, j, n);
  append_row<D>(ap, rt, n, j, hkv);
}

// ---- a decode step over a cache of codes -----------------------------------------
//
// The decode kernel attends to each row's cached tokens only.  The merge
// kernel then codes the row's new token under the scales of its slot's block
// (the append's quantizer, codes.h), adds it to the row's merge as one more
// piece (weight sum 1, its value row the codes' values times the scale), and
// where the slot is the row's next position stores the codes and moves the
// row forward.  A slot outside the pool has no block whose scales could code
// the token: that row attends its cached tokens only and stays as it is.

struct CodeStepArgs {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const uint16_t* k_new;   // [rows][Hkv][D] bf16
  const uint16_t* v_new;
  const int32_t* slots;    // the caller's slot of each row's new token (read here only for rows without tiles)
  const float* scales;     // [num_blocks][Hkv][2]: key scale, value scale
  int32_t* block_tables;
  int32_t* context_lens;
  int max_blocks, block_size, num_blocks;
};

template <int D>
struct NewTokenPiece {
  static constexpr bool kOn = true;
  bool has;            // the slot lies in the pool: the token is attended
  float m[4];          // its base-2 scores for heads wave, wave + 4, ...
  float v[D / 64];     // its value elements lane + 64 e (code value times scale)
  const float* whole;  // whole-segment records [rows][Hkv][g] x (D + 4)
  // the score of head wave + 4 hi; selects, not an indexed read (which would
  // move the object out of registers)
  __device__ __forceinline__ float score(int hi) const {
    return hi == 0 ? m[0] : (hi == 1 ? m[1] : (hi == 2 ? m[2] : m[3]));
  }
};

template <int D, bool I8>
__global__ __launch_bounds__(256) void merge_step8(const float* __restrict__ rec, const float* __restrict__ whole,
                                                   const int32_t* __restrict__ prefix,
                                                   const int32_t* __restrict__ lens,
                                                   const int32_t* __restrict__ row_slots, const uint16_t* __restrict__ q,
                                                   uint16_t* __restrict__ out, int n_seqs, int hq, int hkv, int g,
                                                   int64_t total_waves, float scale_log2, CodeStepArgs a) {
  constexpr int E = D / 64;
  const int j = blockIdx.x;
  const int n = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int B = a.block_size;
  // Every load that does not depend on the slot is issued first, together:
  // the coding below branches, and loads placed after it would each wait
  // out a memory latency of their own.
  const bool has_tiles = prefix[n + 1] > prefix[n];
  const int packed = lens[n];
  const int copied_slot = row_slots[n];
  const int64_t src = (static_cast<int64_t>(n) * hkv + j) * D;
  uint32_t kb[E], vb[E], qb[4][E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kb[e] = a.k_new[src + lane + 64 * e];
    vb[e] = a.v_new[src + lane + 64 * e];
  }
  const uint16_t* qrow = q + (static_cast<int64_t>(n) * hq + j * g) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = min(wave + 4 * i, g - 1);  // heads past g load a valid row and are never used
#pragma unroll
    for (int e = 0; e < E; ++e) qb[i][e] = qrow[h * D + lane + 64 * e];
  }
  // the decode kernel copied the slot of every row with a cached token; a row
  // without one had no tile, so its slot comes from the caller's array
  const int slot = has_tiles ? copied_slot : a.slots[n];
  const bool in_pool = slot >= 0 && static_cast<int64_t>(slot) < static_cast<int64_t>(a.num_blocks) * B;
  const int64_t head = static_cast<int64_t>(in_pool ? slot / B : 0) * hkv + j;
  const float2 kvs = *reinterpret_cast<const float2*>(a.scales + 2 * head);
  const float ks = kvs.x, vs = kvs.y;
  // the lane's elements d = lane + 64 e of the token, coded as the append codes them
  uint32_t kc[E], vc[E];
  float kv[E];
  NewTokenPiece<D> x;
  x.has = in_pool;
  x.whole = whole;
  // all quotients first (their fp64 divisions overlap), then the codes
  double kq[E], vq[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kq[e] = code8_quotient<I8>(bf16_bits_to_f32(kb[e]), ks);
    vq[e] = code8_quotient<I8>(bf16_bits_to_f32(vb[e]), vs);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) {
    kc[e] = code8_encode<I8>(kq[e], bf16_bits_to_f32(kb[e]), ks);
    vc[e] = code8_encode<I8>(vq[e], bf16_bits_to_f32(vb[e]), vs);
    kv[e] = code8_value<I8>(kc[e]);
    x.v[e] = code8_value<I8>(vc[e]) * vs;
  }
  // scores: q . (key codes' values), times scale * log2(e) * key scale, as the decode kernel forms them;
  // only for the heads this wave merges (wave, wave + 4, ... below g)
  const float sk = scale_log2 * ks;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x.m[i] = 0.f;
    if (wave + 4 * i < g) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) dot += bf16_bits_to_f32(qb[i][e]) * kv[e];
      x.m[i] = wave_sum(dot) * sk;
    }
  }
  merge_segment<D, NewTokenPiece<D>>(rec, prefix, out, n_seqs, hq, hkv, g, g, total_waves, j, n, x);
  // store the codes and move the row on where the slot is the row's next position
  const int S0 = pool_tokens(packed);
  if (!(next_fits(packed) && in_pool && slot % B == S0 % B) || wave != 0) return;
  const int64_t pb = slot / B;
  const int off = slot % B;
  const int64_t hd = pb * hkv + j;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t at = (hd * B + off) * D + lane + 64 * e;
    a.k_pool[at] = static_cast<uint8_t>(kc[e]);
    a.v_pool[at] = static_cast<uint8_t>(vc[e]);
  }
  if (j == 0 && lane == 0) {  // the only thread that reads or writes the row
    const int pos = a.context_lens[n];
    a.block_tables[static_cast<int64_t>(n) * a.max_blocks + pos / B] = static_cast<int32_t>(pb);
    a.context_lens[n] = pos + 1;
  }
}

// Both kernels of one decode on stream s.
template <int D, int B, int KV>
void launch_stream_db(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v,
                      const int32_t* bt, const int32_t* cl, void* out, void* ws, int n, int hq, int hkv,
                      int max_blocks, int num_blocks, float scale_log2, const StepInputs* step,
                      const float* scales) {
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
  const int64_t total_waves = static_cast<int64_t>(p.workgroups) * kSW;
  if constexpr (KV != kKvBf16) {
    if (step) {  // the decode attends the cached tokens; the merge kernel adds, codes and stores the new token
      float* whole = reinterpret_cast<float*>(base + p.whole_offset);
      int32_t* lens_ws = reinterpret_cast<int32_t*>(base + p.lens_offset);
      decode_stream<D, B, KV><<<dim3(p.workgroups), dim3(256), p.lds_bytes, s>>>(
          static_cast<const uint16_t*>(q), k, v, bt, cl, static_cast<uint16_t*>(out), rec, prefix, n, hq, hkv, g,
          max_blocks, num_blocks, scale_log2, nullptr, nullptr, step->slots, slots_ws, scales, whole,
          lens_ws);
      CodeStepArgs ca{};
      ca.k_pool = static_cast<uint8_t*>(const_cast<void*>(k));
      ca.v_pool = static_cast<uint8_t*>(const_cast<void*>(v));
      ca.k_new = static_cast<const uint16_t*>(step->k_new);
      ca.v_new = static_cast<const uint16_t*>(step->v_new);
      ca.slots = step->slots;
      ca.scales = scales;
      ca.block_tables = const_cast<int32_t*>(bt);
      ca.context_lens = const_cast<int32_t*>(cl);
      ca.max_blocks = max_blocks;
      ca.block_size = B;
      ca.num_blocks = num_blocks;
      merge_step8<D, KV == kKvInt8><<<dim3(hkv, n), dim3(256), 0, s>>>(
          rec, whole, prefix, lens_ws, slots_ws, static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out), n, hq,
          hkv, g, total_waves, scale_log2, ca);
      return;
    }
  }
  decode_stream<D, B, KV><<<dim3(p.workgroups), dim3(256), p.lds_bytes, s>>>(
      static_cast<const uint16_t*>(q), k, v, bt, cl, static_cast<uint16_t*>(out), rec, prefix, n, hq, hkv, g,
      max_blocks, num_blocks, scale_log2, ap.k_new, ap.v_new, slots_in, slots_ws, scales, nullptr, nullptr);
  merge_stream<D><<<dim3(hkv, n), dim3(256), 0, s>>>(rec, prefix, static_cast<uint16_t*>(out), n, hq, hkv, g,
                                                     total_waves, ap);
}

}  // namespace
}  // namespace pa

// Paged decode attention for gfx950 (MI355X) and its C entry point.
//
// What is computed ("PagedAttention: Virtual Memory for the KV Cache",
// sections 1 and 13; "PagedAttention in vLLM: scattered memory, exact
// attention", sections 10-11): for each sequence n and query head h, with KV
// head j = h / G (G = Hq / Hkv), out = softmax(scale * q K^T) V over the S
// cached tokens, K and V gathered block by block through the block table.
//
// Structure
//   * The context of a sequence is cut into partitions of `part` tokens.  One
//     workgroup handles one (partition, KV head, sequence) and all G query
//     heads of that KV head, so every key/value byte is read once.
//   * Inside a partition the running maximum, shifted weight sum and shifted
//     value sum are updated tile by tile (the online form of section 13 of the
//     first page).  Scores are kept in base 2 (s * log2 e).
//   * If a sequence has one partition its workgroup writes the output
//     directly; otherwise each partition stores its (m, z, u) summary in the
//     workspace and `merge_partitions` combines them with the common-maximum
//     rule of section 11 of the second page, in partition order.
//
// Two kernels compute a partition:
//   decode_mfma   bf16, D in {64, 128}, G <= 16.  q.K^T and P.V run on the
//                 matrix cores (v_mfma_f32_16x16x32_bf16): the G query heads
//                 of a KV head form the N = 16 side (padded), 16 tokens of a
//                 block the M side, d_head the contraction; P.V contracts over
//                 32 tokens.  4 waves per workgroup split the partition's
//                 32-token tiles; their summaries are merged through LDS.
//   decode_generic fp32 or bf16, any G: one wave per (partition, query head,
//                 sequence); per-token dot products with wave reductions.
//
// Pool layout (per layer): K and V [num_blocks][Hkv][B][D].

#include <mutex>

#include "common.h"
#include "decode_stream.h"
#include "decode_tile.h"

namespace pa {
namespace {

constexpr int kWaves = 4;       // waves per workgroup in decode_mfma
constexpr int kTile = 32;       // tokens per wave iteration in decode_mfma
constexpr int kGenericPart = 256;

struct Plan {
  bool mfma;
  int part;   // tokens per partition
  int p_max;  // partitions of the longest sequence
};

inline int ceil_div(int64_t a, int64_t b) { return static_cast<int>((a + b - 1) / b); }

bool mfma_eligible(int g, int d, int block_size, int dtype) {
  return dtype == PA_BF16 && (d == 64 || d == 128) && g >= 1 && g <= 16 &&
         (block_size == 8 || block_size == 16 || block_size == 32);
}

// Partition size: the largest of 512, 256, 128 tokens that still yields at
// least ~2048 workgroups (8 per CU over 256 CUs) for the longest sequence,
// capped so that a partition spans at most 64 blocks (one table entry per
// lane).  A caller of pa_decode_partitioned may fix it instead (`part_tokens`,
// a multiple of 128 up to that cap; 0 = this rule).
Plan make_plan(int num_seqs, int hq, int hkv, int d, int block_size, int max_ctx, int dtype, int part_tokens = 0) {
  Plan p{};
  const int g = hkv > 0 ? hq / hkv : 0;
  p.mfma = mfma_eligible(g, d, block_size, dtype);
  if (p.mfma) {
    int part = 128;
    const int cap = 64 * block_size;
    for (int cand : {512, 256, 128}) {
      if (cand > cap) continue;
      const int64_t wgs = static_cast<int64_t>(num_seqs) * hkv * ceil_div(max_ctx > 0 ? max_ctx : 1, cand);
      part = cand;
      if (wgs >= 2048) break;
    }
    if (part_tokens > 0) part = part_tokens;
    p.part = part;
  } else {
    p.part = kGenericPart;
  }
  p.p_max = max_ctx > 0 ? ceil_div(max_ctx, p.part) : 1;
  return p;
}

size_t plan_workspace_bytes(const Plan& p, int num_seqs, int hq, int d) {
  if (p.p_max <= 1) return 0;
  return static_cast<size_t>(num_seqs) * hq * p.p_max * (d + 2) * sizeof(float);
}

// ---------------------------------------------------------------------------
// decode_mfma
// ---------------------------------------------------------------------------
//
// Lane roles (lane = 16 * gq + r, gq in 0..3, r in 0..15), per 32-token tile
// made of two 16-token slabs a = 0, 1:
//   q.K^T  S^T[token][head] = K[token][:] . Q[head][:]
//          A operand (16 x 32): lane holds key row r of the slab, d-chunk
//          c = 4 jj + gq (8 elements, one 16-byte load from the key row);
//          B operand (32 x 16): Q[head r][chunk c], zero for r >= G;
//          result: lane holds S^T[tokens 4 gq .. 4 gq + 3][head r].
//   P.V    O^T[d][head] += V^T[d][tokens] . P^T[tokens][head]
//          A operand: V^T[d = 16 mm + r][8 tokens] = 4 tokens of slab 0 and 4
//          of slab 1 at rows 4 gq .. 4 gq + 3: the wave copies the tile's 32
//          value rows into its LDS buffer (16 bytes per lane, chunks swizzled
//          as the persistent kernel stages them) and reads each 4-token group
//          back with one transposing 8-byte read;
//          B operand: P^T for those 8 tokens and head r -- exactly the 8
//          scores this lane already holds, so P needs no data movement;
//          result: lane holds O^T[d = 16 mm + 4 gq + i][head r].
// P is split into a bf16 high part and a bf16 residual so that P.V keeps
// about 16 mantissa bits of each weight.
template <int D, int B>
__global__ __launch_bounds__(256) void decode_mfma(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_pool, const uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, uint16_t* __restrict__ out,
    float* __restrict__ ws, int hq, int hkv, int g, int max_blocks, int num_blocks, int part, int p_max,
    float scale_log2) {
  constexpr int X = 8;            // bf16 elements per 16 bytes
  constexpr int KCH = D / 32;     // MFMA steps over d in q.K^T
  constexpr int VT = D / 16;      // output tiles over d in P.V
  constexpr int64_t BLK = static_cast<int64_t>(D) * B;  // elements per (block, KV head)

  // [kWaves][16] m, [kWaves][16] z, then one region per wave of max(g D, 16 D) floats: the wave's staged value
  // rows ([32][D] bf16) while it computes tiles, its summary values ([g][D] fp32) once it is done
  extern __shared__ float lds[];
  const int wreg = (g > 16 ? g : 16) * D;  // floats per wave region

  const int part_id = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int S = context_lens[seq];
  const int tok0 = part_id * part;
  // a length beyond the launch bound (caller error) is cut at p_max partitions
  const int n_parts = S > 0 ? min((S + part - 1) / part, p_max) : 0;

  if (tok0 >= S) {
    if (S <= 0 && part_id == 0) {  // empty context: defined as zeros
      for (int e = threadIdx.x; e < g * D; e += blockDim.x)
        out[(static_cast<int64_t>(seq) * hq + kvh * g) * D + e] = 0;
    }
    return;
  }

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int r = lane & 15;
  const int gq = lane >> 4;

  // block ids of this partition: lane i holds entry (first block + i)
  const int lb0 = tok0 / B;
  const int nb_part = min(min(part / B, (S + B - 1) / B - lb0), max_blocks - lb0);
  int tbl = 0;
  if (lane < nb_part) tbl = block_tables[static_cast<int64_t>(seq) * max_blocks + lb0 + lane];

  // Q operand: head r of this KV head's group, chunks c = 4 jj + gq
  bf16x8 qop[KCH];
  {
    const uint16_t* qh = q + (static_cast<int64_t>(seq) * hq + kvh * g + r) * D;
#pragma unroll
    for (int jj = 0; jj < KCH; ++jj) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < g) v = *reinterpret_cast<const uint4*>(qh + (4 * jj + gq) * X);
      qop[jj] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 acc[VT];
#pragma unroll
  for (int mm = 0; mm < VT; ++mm) acc[mm] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -__FLT_MAX__;  // finite: a tile with no token keeps every exponent finite
  float z_run = 0.f;

  const int tiles = min(part, S - tok0 + kTile - 1) / kTile;  // tiles holding >= 1 valid token
  constexpr int RB = D * 2;                // bytes of one value row
  constexpr int RPP = 1024 / RB;           // rows per 1 KiB of the staging buffer
  unsigned char* vst = reinterpret_cast<unsigned char*>(lds + 2 * kWaves * 16 + wave * wreg);
  const int vj = r >> 2, vq = r & 3;       // the value row / d quarter this lane points at in a transposing read
  const uint16_t* kh = k_pool + static_cast<int64_t>(kvh) * BLK;
  const uint16_t* vh = v_pool + static_cast<int64_t>(kvh) * BLK;
  const int64_t blk_stride = static_cast<int64_t>(hkv) * BLK;

  for (int tile = wave; tile < tiles; tile += kWaves) {
    const int t0 = tok0 + tile * kTile;

    // ---- loads -------------------------------------------------------------
    bf16x8 kop[2][KCH];
    bf16x8 vop[VT];
    uint2 vlo[VT], vhi[VT];
    bool blk_ok[2];  // the block of the lane's 4-token group of slab a lies in the pool
    // value rows t0 .. t0 + 31 into this wave's LDS buffer (zeros where the
    // token is past the end or its block outside the pool)
#pragma unroll
    for (int p = 0; p < kTile * RB / 1024; ++p) {
      const int row = p * RPP + lane * 16 / RB;
      const int slot = (lane * 16 % RB) / 16;
      const int tv = t0 + row;
      const int pbv = __shfl(tbl, (tv / B) - lb0);
      uint4 v = make_uint4(0, 0, 0, 0);
      if (tv < S && pbv >= 0 && pbv < num_blocks)
        v = load_kv16(vh + static_cast<int64_t>(pbv) * blk_stride + (tv % B) * D +
                      ((slot ^ stage_swz<D, false>(row)) << 3));
      *reinterpret_cast<uint4*>(vst + p * 1024 + lane * 16) = v;
    }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      // key row r of slab a
      const int tk = t0 + 16 * a + r;
      const int pbk = __shfl(tbl, (tk / B) - lb0);
      const bool kval = tk < S && pbk >= 0 && pbk < num_blocks;
      const uint16_t* kb = kh + static_cast<int64_t>(pbk) * blk_stride + (tk % B) * D;
#pragma unroll
      for (int jj = 0; jj < KCH; ++jj) {
        uint4 v = make_uint4(0, 0, 0, 0);
        if (kval) v = load_kv16(kb + (4 * jj + gq) * X);
        kop[a][jj] = __builtin_bit_cast(bf16x8, v);
      }
      const int tv = t0 + 16 * a + 4 * gq;
      blk_ok[a] = [&] {
        const int pbv = __shfl(tbl, (tv / B) - lb0);
        return pbv >= 0 && pbv < num_blocks;
      }();
    }
    // the wave's own LDS writes above are done before its reads below (LDS
    // instructions of one wave execute in order; the compiler keeps the order)
    __asm__ volatile("" ::: "memory");
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const int row = 16 * a + 4 * gq + vj;
      const int sv = stage_swz<D, false>(row);
#pragma unroll
      for (int mm = 0; mm < VT; ++mm) {
        const uint2 v = lds_read_tr16(vst + row * RB + (((2 * mm + (vq >> 1)) ^ sv) << 4) + (vq & 1) * 8);
        if (a == 0) vlo[mm] = v; else vhi[mm] = v;
      }
    }
    __asm__ volatile("" ::: "memory");
    // zero the value elements of tokens past the end (a stale or NaN slot
    // must not reach P.V: 0 * NaN is NaN)
    {
      const int tv0 = t0 + 4 * gq;
      const int tv1 = t0 + 16 + 4 * gq;
      const int n0 = min(max(S - tv0, 0), 4);
      const int n1 = min(max(S - tv1, 0), 4);
      const uint32_t m0a = n0 >= 2 ? 0xffffffffu : (n0 == 1 ? 0x0000ffffu : 0u);
      const uint32_t m0b = n0 >= 4 ? 0xffffffffu : (n0 == 3 ? 0x0000ffffu : 0u);
      const uint32_t m1a = n1 >= 2 ? 0xffffffffu : (n1 == 1 ? 0x0000ffffu : 0u);
      const uint32_t m1b = n1 >= 4 ? 0xffffffffu : (n1 == 3 ? 0x0000ffffu : 0u);
#pragma unroll
      for (int mm = 0; mm < VT; ++mm) {
        uint4 w = make_uint4(vlo[mm].x & m0a, vlo[mm].y & m0b, vhi[mm].x & m1a, vhi[mm].y & m1b);
        vop[mm] = __builtin_bit_cast(bf16x8, w);
      }
    }

    // ---- scores: S^T = K . Q^T --------------------------------------------
    f32x4 s[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      s[a] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < KCH; ++jj)
        s[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[a][jj], qop[jj], s[a], 0, 0, 0);
    }

    // ---- online softmax (base 2) -------------------------------------------
    float x[2][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tok = t0 + 16 * a + 4 * gq + i;
        x[a][i] = tok < S && blk_ok[a] ? s[a][i] * scale_log2 : -INFINITY;  // out-of-pool tokens left out
        tmax = fmaxf(tmax, x[a][i]);
      }
    tmax = max_across_groups(tmax);
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
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
    z_run = z_run * alpha + psum;

    // ---- O^T += V^T . P^T ------------------------------------------------------
#pragma unroll
    for (int mm = 0; mm < VT; ++mm) {
      acc[mm] *= alpha;
      acc[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[mm], phi, acc[mm], 0, 0, 0);
      acc[mm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop[mm], plo, acc[mm], 0, 0, 0);
    }
  }

  // ---- merge the 4 waves through LDS -----------------------------------------
  z_run = sum_across_groups(z_run);
  // the wave's region now holds its summary values (its own tiles are done: no other wave reads it before the barrier)
  __asm__ volatile("" ::: "memory");
  float* lds_m = lds;                         // [kWaves][16]
  float* lds_z = lds_m + kWaves * 16;         // [kWaves][16]
  float* lds_u = lds_z + kWaves * 16;         // [kWaves][wreg]: [g][D] used
  if (r < g) {
#pragma unroll
    for (int mm = 0; mm < VT; ++mm)
      *reinterpret_cast<f32x4*>(lds_u + wave * wreg + r * D + 16 * mm + 4 * gq) = acc[mm];
    if (gq == 0) {
      lds_m[wave * 16 + r] = m_run;
      lds_z[wave * 16 + r] = z_run;
    }
  }
  __syncthreads();

  const int64_t head0 = static_cast<int64_t>(seq) * hq + kvh * g;
  for (int e = threadIdx.x; e < g * D; e += blockDim.x) {
    const int h = e / D;
    const int dd = e - h * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, lds_m[w * 16 + h]);
    float zz = 0.f, uu = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(lds_m[w * 16 + h] - mx);  // 0 for idle waves (maximum: the most negative float)
      zz += f * lds_z[w * 16 + h];
      uu += f * lds_u[w * wreg + h * D + dd];
    }
    if (n_parts == 1) {
      out[(head0 + h) * D + dd] = f32_to_bf16_bits(zz > 0.f ? uu / zz : 0.f);  // no token at all: zeros
    } else {
      const int64_t row = (head0 + h) * p_max + part_id;
      const int64_t n_rows = static_cast<int64_t>(gridDim.z) * hq * p_max;
      ws[2 * n_rows + row * D + dd] = uu;
      if (dd == 0) {
        ws[row] = mx;
        ws[n_rows + row] = zz;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// decode_generic: one wave per (partition, query head, sequence)
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_generic(
    const T* __restrict__ q, const T* __restrict__ k_pool, const T* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ context_lens, T* __restrict__ out,
    float* __restrict__ ws, int hq, int hkv, int block_size, int max_blocks, int num_blocks, int part, int p_max,
    float scale_log2) {
  constexpr int E = D / 64;  // elements per lane
  const int part_id = blockIdx.x;
  const int h = blockIdx.y;
  const int seq = blockIdx.z;
  const int g = hq / hkv;
  const int kvh = h / g;
  const int S = context_lens[seq];
  const int tok0 = part_id * part;
  const int lane = threadIdx.x;
  const int64_t orow = (static_cast<int64_t>(seq) * hq + h) * D;
  if (tok0 >= S) {
    if (S <= 0 && part_id == 0)
      for (int e = 0; e < E; ++e) Elem<T>::store(out + orow + lane + 64 * e, 0.f);
    return;
  }
  const int tok1 = min(S, tok0 + part);
  const int n_parts = min((S + part - 1) / part, p_max);

  float qv[E], u[E];
  for (int e = 0; e < E; ++e) {
    qv[e] = Elem<T>::load(q + orow + lane + 64 * e);
    u[e] = 0.f;
  }
  float m_run = -__FLT_MAX__, z_run = 0.f;  // finite: a block outside the pool first keeps exponents finite
  const int64_t blk_stride = static_cast<int64_t>(hkv) * D * block_size;
  for (int t = tok0; t < tok1; ++t) {
    const int lb = t / block_size;
    const int pb = lb < max_blocks ? block_tables[static_cast<int64_t>(seq) * max_blocks + lb] : -1;
    const int off = t % block_size;
    const bool ok = pb >= 0 && pb < num_blocks;
    const T* kb = k_pool + static_cast<int64_t>(pb) * blk_stride + static_cast<int64_t>(kvh) * D * block_size;
    const T* vb = v_pool + static_cast<int64_t>(pb) * blk_stride + static_cast<int64_t>(kvh) * D * block_size;
    float dot = 0.f;
    float vv[E];
    for (int e = 0; e < E; ++e) {
      const int d = lane + 64 * e;
      const float kx = ok ? Elem<T>::load(kb + off * D + d) : 0.f;
      vv[e] = ok ? Elem<T>::load(vb + off * D + d) : 0.f;
      dot += qv[e] * kx;
    }
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) dot += __shfl_xor(dot, sh);
    const float s2 = ok ? dot * scale_log2 : -INFINITY;  // a block outside the pool is left out
    const float m_new = fmaxf(m_run, s2);
    const float alpha = exp2f(m_run - m_new);
    const float p = exp2f(s2 - m_new);
    z_run = z_run * alpha + p;
    for (int e = 0; e < E; ++e) u[e] = u[e] * alpha + p * vv[e];
    m_run = m_new;
  }
  if (n_parts == 1) {
    for (int e = 0; e < E; ++e) Elem<T>::store(out + orow + lane + 64 * e, z_run > 0.f ? u[e] / z_run : 0.f);
  } else {
    const int64_t row = (static_cast<int64_t>(seq) * hq + h) * p_max + part_id;
    const int64_t n_rows = static_cast<int64_t>(gridDim.z) * hq * p_max;
    for (int e = 0; e < E; ++e) ws[2 * n_rows + row * D + lane + 64 * e] = u[e];
    if (lane == 0) {
      ws[row] = m_run;
      ws[n_rows + row] = z_run;
    }
  }
}

// ---------------------------------------------------------------------------
// merge_partitions: common-maximum merge of the partition summaries,
// partitions combined in index order.  One workgroup of D threads per
// (query head, sequence); sequences with a single partition were finished by
// the decode kernel.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(D) void merge_partitions(const float* __restrict__ ws,
                                                      const int32_t* __restrict__ context_lens, T* __restrict__ out,
                                                      int num_seqs, int hq, int part, int p_max) {
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const int S = context_lens[seq];
  const int n_parts = S > 0 ? min((S + part - 1) / part, p_max) : 0;
  if (n_parts <= 1) return;
  const int64_t n_rows = static_cast<int64_t>(num_seqs) * hq * p_max;
  const int64_t row0 = (static_cast<int64_t>(seq) * hq + h) * p_max;
  const int dd = threadIdx.x;
  float mx = -INFINITY;
  for (int p = 0; p < n_parts; ++p) mx = fmaxf(mx, ws[row0 + p]);
  float zz = 0.f, uu = 0.f;
  for (int p = 0; p < n_parts; ++p) {
    const float f = __builtin_amdgcn_exp2f(ws[row0 + p] - mx);
    zz += f * ws[n_rows + row0 + p];
    uu += f * ws[2 * n_rows + (row0 + p) * D + dd];
  }
  Elem<T>::store(out + (static_cast<int64_t>(seq) * hq + h) * D + dd, zz > 0.f ? uu / zz : 0.f);
}

template <int D, int B>
void launch_mfma(const Plan& pl, dim3 grid, size_t lds, hipStream_t s, const void* q, const void* k, const void* v,
                 const int32_t* bt, const int32_t* cl, void* out, float* ws, int hq, int hkv, int g, int max_blocks,
                 int num_blocks, float scale_log2) {
  decode_mfma<D, B><<<grid, dim3(256), lds, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), bt, cl,
      static_cast<uint16_t*>(out), ws, hq, hkv, g, max_blocks, num_blocks, pl.part, pl.p_max, scale_log2);
}

template <int D>
void launch_mfma_b(int block_size, const Plan& pl, dim3 grid, size_t lds, hipStream_t s, const void* q,
                   const void* k, const void* v, const int32_t* bt, const int32_t* cl, void* out, float* ws, int hq,
                   int hkv, int g, int max_blocks, int num_blocks, float scale_log2) {
  switch (block_size) {
    case 8: launch_mfma<D, 8>(pl, grid, lds, s, q, k, v, bt, cl, out, ws, hq, hkv, g, max_blocks, num_blocks, scale_log2); break;
    case 16: launch_mfma<D, 16>(pl, grid, lds, s, q, k, v, bt, cl, out, ws, hq, hkv, g, max_blocks, num_blocks, scale_log2); break;
    default: launch_mfma<D, 32>(pl, grid, lds, s, q, k, v, bt, cl, out, ws, hq, hkv, g, max_blocks, num_blocks, scale_log2); break;
  }
}

template <typename T, int D>
void launch_generic(const Plan& pl, dim3 grid, hipStream_t s, const void* q, const void* k, const void* v,
                    const int32_t* bt, const int32_t* cl, void* out, float* ws, int hq, int hkv, int block_size,
                    int max_blocks, int num_blocks, float scale_log2) {
  decode_generic<T, D><<<grid, dim3(64), 0, s>>>(static_cast<const T*>(q), static_cast<const T*>(k),
                                                 static_cast<const T*>(v), bt, cl, static_cast<T*>(out), ws, hq, hkv,
                                                 block_size, max_blocks, num_blocks, pl.part, pl.p_max, scale_log2);
}

template <typename T, int D>
void launch_merge(const Plan& pl, hipStream_t s, const float* ws, const int32_t* cl, void* out, int num_seqs, int hq) {
  merge_partitions<T, D><<<dim3(hq, num_seqs), dim3(D), 0, s>>>(ws, cl, static_cast<T*>(out), num_seqs, hq, pl.part,
                                                                pl.p_max);
}

}  // namespace
}  // namespace pa

namespace pa {
namespace {
// The persistent stream kernel serves bf16 with G <= 16 and N <= 3072; the
// partitioned kernels serve the rest (and pa_decode_partitioned).
bool use_stream(int num_seqs, int hq, int hkv, int d, int block_size, int dtype) {
  if (hkv <= 0 || hq % hkv != 0) return false;
  return stream_eligible(num_seqs, hq / hkv, d, block_size, dtype);
}
// Partition sizes a caller may fix: multiples of 128 tokens spanning at most
// 64 blocks (0 = automatic).
bool valid_part_tokens(int part_tokens, int block_size) {
  return part_tokens == 0 || (part_tokens >= 128 && part_tokens % 128 == 0 && part_tokens <= 64 * block_size);
}
// Groups are served by the shared-prefix kernel where the persistent kernel
// runs and the sizes fit it; elsewhere they are ignored, which gives the same
// attention.
bool use_shared(int num_seqs, int num_groups, int hq, int hkv, int d, int block_size, int dtype) {
  return num_groups > 0 && use_stream(num_seqs, hq, hkv, d, block_size, dtype) &&
         shared_eligible(num_seqs, num_groups, hq / hkv, d, block_size, dtype);
}
}  // namespace
}  // namespace pa

extern "C" size_t pa_decode_workspace_bytes(int num_seqs, int Hq, int Hkv, int d_head, int block_size,
                                            int max_context_len, int dtype) {
  if (num_seqs <= 0 || Hq <= 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0 || max_context_len < 0) return 0;
  if (dtype == PA_FP8_E4M3 || dtype == PA_INT8) {  // one-byte codes: 64-token tiles
    if (Hq % Hkv != 0 || !pa::stream_eligible_fp8(num_seqs, Hq / Hkv, d_head, block_size)) return 0;
    return pa::stream_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, true).workspace_bytes;
  }
  if (pa::use_stream(num_seqs, Hq, Hkv, d_head, block_size, dtype))
    return pa::stream_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len).workspace_bytes;
  const pa::Plan p = pa::make_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype);
  return pa::plan_workspace_bytes(p, num_seqs, Hq, d_head);
}

extern "C" size_t pa_decode_shared_workspace_bytes(int num_seqs, int num_groups, int Hq, int Hkv, int d_head,
                                                   int block_size, int max_context_len, int dtype) {
  if (num_seqs <= 0 || num_groups < 0 || Hq <= 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0 ||
      max_context_len < 0 || Hq % Hkv != 0 || dtype == PA_FP8_E4M3)
    return 0;
  if (pa::use_shared(num_seqs, num_groups, Hq, Hkv, d_head, block_size, dtype))
    return pa::shared_plan(num_seqs, num_groups, Hq, Hkv, d_head, block_size, max_context_len).workspace_bytes;
  return pa_decode_workspace_bytes(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype);
}

extern "C" size_t pa_decode_partitioned_workspace_bytes(int num_seqs, int Hq, int Hkv, int d_head, int block_size,
                                                        int max_context_len, int dtype, int partition_tokens) {
  if (num_seqs <= 0 || Hq <= 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0 || max_context_len < 0) return 0;
  if (Hq % Hkv != 0 || (dtype != PA_F32 && dtype != PA_BF16)) return 0;
  if (!pa::valid_part_tokens(partition_tokens, block_size)) return 0;
  const pa::Plan p = pa::make_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype, partition_tokens);
  return pa::plan_workspace_bytes(p, num_seqs, Hq, d_head);
}

extern "C" int pa_decode_partition_tokens(int num_seqs, int Hq, int Hkv, int d_head, int block_size,
                                          int max_context_len, int dtype) {
  if (num_seqs <= 0 || Hq <= 0 || Hkv <= 0) return 0;
  if (dtype == PA_FP8_E4M3) return 0;
  if (pa::use_stream(num_seqs, Hq, Hkv, d_head, block_size, dtype)) return 0;
  return pa::make_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype).part;
}

namespace {
int decode_impl(void* out, const void* q, const void* k_pool, const void* v_pool, const int32_t* block_tables,
                const int32_t* context_lens, int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                int max_blocks_per_seq, int max_context_len, int num_blocks, int dtype, void* workspace,
                size_t workspace_bytes, void* stream, const pa::StepInputs* step, const int32_t* groups = nullptr,
                int num_groups = 0, bool partitioned = false, int part_tokens = 0) {
  using namespace pa;
  if (num_seqs < 0 || Hq <= 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
      max_context_len < 0 || num_blocks < 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size < max_context_len) return PA_ERR_INVALID_ARG;
  if (!(d_head == 64 || d_head == 128) || !(block_size == 8 || block_size == 16 || block_size == 32) ||
      Hq / Hkv > 64)
    return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (num_blocks < 1 || max_blocks_per_seq < 1) return PA_ERR_INVALID_ARG;  // kernels may read block 0 / entry 0
  if (num_seqs > 65535 || Hq > 65535) return PA_ERR_UNSUPPORTED;

  const float scale_log2_s = scale * kLog2e;
  if (num_groups < 0 || (num_groups > 0 && !groups)) return PA_ERR_INVALID_ARG;
  if (partitioned && (step || num_groups > 0 || !valid_part_tokens(part_tokens, block_size))) return PA_ERR_INVALID_ARG;
  if (!partitioned && use_shared(num_seqs, num_groups, Hq, Hkv, d_head, block_size, dtype)) {
    const StreamPlan sp = shared_plan(num_seqs, num_groups, Hq, Hkv, d_head, block_size, max_context_len);
    if (!workspace || workspace_bytes < sp.workspace_bytes) return PA_ERR_WORKSPACE;
    return launch_shared(sp, static_cast<hipStream_t>(stream), q, k_pool, v_pool, block_tables, context_lens, groups,
                         num_groups, out, workspace, num_seqs, Hq, Hkv, d_head, block_size, max_blocks_per_seq,
                         num_blocks, scale_log2_s, step);
  }
  if (!partitioned && use_stream(num_seqs, Hq, Hkv, d_head, block_size, dtype)) {
    const StreamPlan sp = stream_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len);
    if (!workspace || workspace_bytes < sp.workspace_bytes) return PA_ERR_WORKSPACE;
    return launch_stream(sp, static_cast<hipStream_t>(stream), q, k_pool, v_pool, block_tables, context_lens, out,
                         workspace, num_seqs, Hq, Hkv, d_head, block_size, max_blocks_per_seq, num_blocks,
                         scale_log2_s, step);
  }
  const Plan pl = make_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, dtype, part_tokens);
  const size_t need = plan_workspace_bytes(pl, num_seqs, Hq, d_head);
  if (need > 0 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  float* ws = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float scale_log2 = scale * kLog2e;
  const int g = Hq / Hkv;

  if (pl.mfma) {
    const dim3 grid(pl.p_max, Hkv, num_seqs);
    const size_t lds = (2 * kWaves * 16 + static_cast<size_t>(kWaves) * (g > 16 ? g : 16) * d_head) * sizeof(float);
    if (d_head == 128)
      launch_mfma_b<128>(block_size, pl, grid, lds, s, q, k_pool, v_pool, block_tables, context_lens, out, ws, Hq,
                         Hkv, g, max_blocks_per_seq, num_blocks, scale_log2);
    else
      launch_mfma_b<64>(block_size, pl, grid, lds, s, q, k_pool, v_pool, block_tables, context_lens, out, ws, Hq,
                        Hkv, g, max_blocks_per_seq, num_blocks, scale_log2);
  } else {
    const dim3 grid(pl.p_max, Hq, num_seqs);
    if (dtype == PA_BF16) {
      if (d_head == 128)
        launch_generic<uint16_t, 128>(pl, grid, s, q, k_pool, v_pool, block_tables, context_lens, out, ws, Hq, Hkv,
                                      block_size, max_blocks_per_seq, num_blocks, scale_log2);
      else
        launch_generic<uint16_t, 64>(pl, grid, s, q, k_pool, v_pool, block_tables, context_lens, out, ws, Hq, Hkv,
                                     block_size, max_blocks_per_seq, num_blocks, scale_log2);
    } else {
      if (d_head == 128)
        launch_generic<float, 128>(pl, grid, s, q, k_pool, v_pool, block_tables, context_lens, out, ws, Hq, Hkv,
                                   block_size, max_blocks_per_seq, num_blocks, scale_log2);
      else
        launch_generic<float, 64>(pl, grid, s, q, k_pool, v_pool, block_tables, context_lens, out, ws, Hq, Hkv,
                                  block_size, max_blocks_per_seq, num_blocks, scale_log2);
    }
  }
  int st = launch_status();
  if (st != PA_OK || pl.p_max <= 1) return st;
  if (dtype == PA_BF16) {
    if (d_head == 128) launch_merge<uint16_t, 128>(pl, s, ws, context_lens, out, num_seqs, Hq);
    else launch_merge<uint16_t, 64>(pl, s, ws, context_lens, out, num_seqs, Hq);
  } else {
    if (d_head == 128) launch_merge<float, 128>(pl, s, ws, context_lens, out, num_seqs, Hq);
    else launch_merge<float, 64>(pl, s, ws, context_lens, out, num_seqs, Hq);
  }
  return launch_status();
}
}  // namespace

extern "C" int pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int Hq, int Hkv,
                         int d_head, int block_size, float scale, int max_blocks_per_seq, int max_context_len,
                         int num_blocks, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, Hq, Hkv, d_head, block_size,
                     scale, max_blocks_per_seq, max_context_len, num_blocks, dtype, workspace, workspace_bytes, stream,
                     nullptr);
}

extern "C" int pa_decode_partitioned(void* out, const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int Hq,
                                     int Hkv, int d_head, int block_size, float scale, int max_blocks_per_seq,
                                     int max_context_len, int num_blocks, int dtype, int partition_tokens,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, Hq, Hkv, d_head, block_size,
                     scale, max_blocks_per_seq, max_context_len, num_blocks, dtype, workspace, workspace_bytes, stream,
                     nullptr, nullptr, 0, true, partition_tokens);
}

extern "C" int pa_decode_step(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                              void* v_pool, const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                              int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                              int max_blocks_per_seq, int max_context_len, int num_blocks, int dtype,
                              void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pa;
  if (num_seqs < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  // served by the persistent bf16 kernel only; other shapes use pa_append_step + pa_decode
  if (!use_stream(num_seqs, Hq, Hkv, d_head, block_size, dtype)) return PA_ERR_UNSUPPORTED;
  const StepInputs step{k_new, v_new, slot_mapping};
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, Hq, Hkv, d_head, block_size,
                     scale, max_blocks_per_seq, max_context_len, num_blocks, dtype, workspace, workspace_bytes,
                     stream, &step);
}

// ---- pa_decode_step_noalloc: the step with its workspace in a fixed device array ----
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid allocation): the workspace of pa_decode_step
// lives in `scratch`, one array per GPU that the library holds until the
// process ends.  Host code never uses the array's name as an address (on the
// host it is a stand-in, not a device pointer): each device's address comes
// from hipGetSymbolAddress, taken once per device with that device current.

namespace {
constexpr size_t kNoAllocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static_assert(kNoAllocScratchBytes % 256 == 0, "scratch is a whole number of 256-byte lines");
}  // namespace

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

// The device address of `scratch` on the current device, or nullptr when the
// runtime cannot give it.  Taken on a device's first call and kept.
void* scratch_on_current_device() {
  constexpr int kMaxDevices = 64;
  static void* ptrs[kMaxDevices] = {};
  static std::mutex mu;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return nullptr;
    }
    ptrs[dev] = ptr;
  }
  return ptrs[dev];
}

}  // namespace

extern "C" int pa_decode_step_noalloc(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                                      void* v_pool, const int32_t* slot_mapping, int32_t* block_tables,
                                      int32_t* context_lens, int num_seqs, int Hq, int Hkv, int d_head,
                                      int block_size, float scale, int max_blocks_per_seq, int max_context_len,
                                      int num_blocks, int dtype, void* stream) {
  using namespace pa;
  if (num_seqs < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || d_head <= 0 || block_size <= 0 || max_context_len < 0)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  if (!use_stream(num_seqs, Hq, Hkv, d_head, block_size, dtype)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  const size_t need = stream_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len).workspace_bytes;
  if (need > kNoAllocScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return PA_ERR_HIP;
  const StepInputs step{k_new, v_new, slot_mapping};
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, Hq, Hkv, d_head, block_size,
                     scale, max_blocks_per_seq, max_context_len, num_blocks, dtype, ws, kNoAllocScratchBytes, stream,
                     &step);
}

extern "C" int pa_decode_shared(void* out, const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* block_tables, const int32_t* context_lens, const int32_t* groups,
                                int num_groups, int num_seqs, int Hq, int Hkv, int d_head, int block_size,
                                float scale, int max_blocks_per_seq, int max_context_len, int num_blocks, int dtype,
                                void* workspace, size_t workspace_bytes, void* stream) {
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, Hq, Hkv, d_head, block_size,
                     scale, max_blocks_per_seq, max_context_len, num_blocks, dtype, workspace, workspace_bytes, stream,
                     nullptr, groups, num_groups);
}

extern "C" int pa_decode_step_shared(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                                     void* v_pool, const int32_t* slot_mapping, int32_t* block_tables,
                                     int32_t* context_lens, const int32_t* groups, int num_groups, int num_seqs,
                                     int Hq, int Hkv, int d_head, int block_size, float scale,
                                     int max_blocks_per_seq, int max_context_len, int num_blocks, int dtype,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  using namespace pa;
  if (num_seqs < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0) return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  if (!use_stream(num_seqs, Hq, Hkv, d_head, block_size, dtype)) return PA_ERR_UNSUPPORTED;
  const StepInputs step{k_new, v_new, slot_mapping};
  return decode_impl(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, Hq, Hkv, d_head, block_size,
                     scale, max_blocks_per_seq, max_context_len, num_blocks, dtype, workspace, workspace_bytes,
                     stream, &step, groups, num_groups);
}

namespace {

// pa_decode over a cache of one-byte codes (FP8 E4M3 or INT8) with scales.
int decode_codes(int codes, void* out, const void* q, const void* k_pool, const void* v_pool, const float* scales,
                 const int32_t* block_tables, const int32_t* context_lens, int num_seqs, int Hq,
                 int Hkv, int d_head, int block_size, float scale, int max_blocks_per_seq, int max_context_len,
                 int num_blocks, void* workspace, size_t workspace_bytes, void* stream,
                 const pa::StepInputs* step = nullptr) {
  using namespace pa;
  if (num_seqs < 0 || Hq <= 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0 || max_blocks_per_seq < 0 ||
      max_context_len < 0 || num_blocks < 0)
    return PA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return PA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(max_blocks_per_seq) * block_size < max_context_len) return PA_ERR_INVALID_ARG;
  if (!stream_eligible_fp8(num_seqs, Hq / Hkv, d_head, block_size) || Hq > 65535) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !scales || !block_tables || !context_lens) return PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(scales) % 8 != 0) return PA_ERR_INVALID_ARG;  // read as (key, value) pairs
  if (num_blocks < 1 || max_blocks_per_seq < 1) return PA_ERR_INVALID_ARG;  // the kernel may read block 0 / entry 0
  const StreamPlan sp = stream_plan(num_seqs, Hq, Hkv, d_head, block_size, max_context_len, true);
  if (!workspace || workspace_bytes < sp.workspace_bytes) return PA_ERR_WORKSPACE;
  return launch_stream(sp, static_cast<hipStream_t>(stream), q, k_pool, v_pool, block_tables, context_lens, out,
                       workspace, num_seqs, Hq, Hkv, d_head, block_size, max_blocks_per_seq, num_blocks,
                       scale * kLog2e, step, scales, codes);
}

int decode_step_codes(int codes, void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                      void* v_pool, const float* scales, const int32_t* slot_mapping,
                      int32_t* block_tables, int32_t* context_lens, int num_seqs, int Hq, int Hkv, int d_head,
                      int block_size, float scale, int max_blocks_per_seq, int max_context_len, int num_blocks,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping)) return PA_ERR_INVALID_ARG;
  const pa::StepInputs step{k_new, v_new, slot_mapping};
  return decode_codes(codes, out, q, k_pool, v_pool, scales, block_tables, context_lens, num_seqs, Hq, Hkv,
                      d_head, block_size, scale, max_blocks_per_seq, max_context_len, num_blocks, workspace,
                      workspace_bytes, stream, &step);
}

}  // namespace

extern "C" int pa_decode_fp8(void* out, const void* q, const void* k_pool, const void* v_pool, const float* scales,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                             int max_blocks_per_seq, int max_context_len, int num_blocks, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return decode_codes(pa::kKvE4m3, out, q, k_pool, v_pool, scales, block_tables, context_lens, num_seqs,
                      Hq, Hkv, d_head, block_size, scale, max_blocks_per_seq, max_context_len, num_blocks, workspace,
                      workspace_bytes, stream);
}

extern "C" int pa_decode_int8(void* out, const void* q, const void* k_pool, const void* v_pool, const float* scales,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                              int max_blocks_per_seq, int max_context_len, int num_blocks, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_codes(pa::kKvInt8, out, q, k_pool, v_pool, scales, block_tables, context_lens, num_seqs,
                      Hq, Hkv, d_head, block_size, scale, max_blocks_per_seq, max_context_len, num_blocks, workspace,
                      workspace_bytes, stream);
}

extern "C" int pa_decode_step_fp8(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                                  void* v_pool, const float* scales,
                                  const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                                  int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                                  int max_blocks_per_seq, int max_context_len, int num_blocks, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return decode_step_codes(pa::kKvE4m3, out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping,
                           block_tables, context_lens, num_seqs, Hq, Hkv, d_head, block_size, scale,
                           max_blocks_per_seq, max_context_len, num_blocks, workspace, workspace_bytes, stream);
}

extern "C" int pa_decode_step_int8(void* out, const void* q, const void* k_new, const void* v_new, void* k_pool,
                                   void* v_pool, const float* scales,
                                   const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                                   int num_seqs, int Hq, int Hkv, int d_head, int block_size, float scale,
                                   int max_blocks_per_seq, int max_context_len, int num_blocks, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return decode_step_codes(pa::kKvInt8, out, q, k_new, v_new, k_pool, v_pool, scales, slot_mapping,
                           block_tables, context_lens, num_seqs, Hq, Hkv, d_head, block_size, scale,
                           max_blocks_per_seq, max_context_len, num_blocks, workspace, workspace_bytes, stream);
}

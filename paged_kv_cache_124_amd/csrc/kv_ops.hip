// KV append and copy-on-write block copy kernels (gfx950) and their C entry
// points, for bf16 / fp32 caches and for a cache of FP8 (E4M3) codes with
// per-(block, KV head) scales.
//
// Append: "PagedAttention: Virtual Memory for the KV Cache", section 16 -- the
// new position's key and value are written into its block at its offset.
// Copy: same page, sections 15-16 -- a shared tail block is cloned before a
// sequence writes into it.  Both are pure data movement and bit-exact.
//
// Pool layout (per layer): K and V [num_blocks][Hkv][B][D] -- each token's
// key (and value) row of one KV head is D contiguous elements.

#include "codes.h"
#include "common.h"

namespace pa {
namespace {

// One thread per (token, KV head, 16-byte chunk of the row): one 16-byte
// store into the key row and one into the value row of the token's slot.
template <typename T>
__global__ __launch_bounds__(256) void append_kv_kernel(T* __restrict__ k_pool, T* __restrict__ v_pool,
                                                        const T* __restrict__ k_new,
                                                        const T* __restrict__ v_new,
                                                        const int32_t* __restrict__ slot_mapping,
                                                        int num_tokens, int hkv, int d, int block_size,
                                                        int64_t num_slots) {
  constexpr int X = 16 / static_cast<int>(sizeof(T));
  const int chunks = d / X;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int c = static_cast<int>(gid % chunks);
  const int64_t th = gid / chunks;
  const int j = static_cast<int>(th % hkv);
  const int64_t t = th / hkv;
  if (t >= num_tokens) return;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t pb = slot / block_size;
  const int off = static_cast<int>(slot % block_size);

  const int64_t src = (t * hkv + j) * d + static_cast<int64_t>(c) * X;
  const int64_t dst = ((pb * hkv + j) * block_size + off) * d + static_cast<int64_t>(c) * X;
  *reinterpret_cast<uint4*>(k_pool + dst) = *reinterpret_cast<const uint4*>(k_new + src);
  *reinterpret_cast<uint4*>(v_pool + dst) = *reinterpret_cast<const uint4*>(v_new + src);
}

// One decode step's append for a batch whose block tables and lengths stay
// resident on the device: token n belongs to sequence row n.  Threads as in
// append_kv_kernel; the thread of (n, head 0, chunk 0) also moves the row
// forward -- block_tables[n][S / B] = slot / B and context_lens[n] = S + 1,
// S being the row's length before the step -- which is what the host block
// manager's table and length become after the same append (the slot's block
// is the table entry of position S, whether the block was in place, fresh
// or a copy-on-write destination).  Only that thread touches the row, so the
// key / value writers never read a length being changed.
template <typename T>
__global__ __launch_bounds__(256) void append_step_kernel(T* __restrict__ k_pool, T* __restrict__ v_pool,
                                                          const T* __restrict__ k_new, const T* __restrict__ v_new,
                                                          const int32_t* __restrict__ slot_mapping,
                                                          int32_t* __restrict__ block_tables,
                                                          int32_t* __restrict__ context_lens, int num_seqs,
                                                          int max_blocks, int hkv, int d, int block_size,
                                                          int64_t num_slots) {
  constexpr int X = 16 / static_cast<int>(sizeof(T));
  const int chunks = d / X;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int c = static_cast<int>(gid % chunks);
  const int64_t th = gid / chunks;
  const int j = static_cast<int>(th % hkv);
  const int64_t n = th / hkv;
  if (n >= num_seqs) return;
  const int64_t slot = slot_mapping[n];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t pb = slot / block_size;
  const int off = static_cast<int>(slot % block_size);
  if (j == 0 && c == 0) {
    const int pos = context_lens[n];
    // a slot that does not sit at the row's next position leaves the row as it is
    if (pos >= 0 && pos / block_size < max_blocks && pos % block_size == off) {
      block_tables[n * max_blocks + pos / block_size] = static_cast<int32_t>(pb);
      context_lens[n] = pos + 1;
    }
  }
  const int64_t src = (n * hkv + j) * d + static_cast<int64_t>(c) * X;
  const int64_t dst = ((pb * hkv + j) * block_size + off) * d + static_cast<int64_t>(c) * X;
  *reinterpret_cast<uint4*>(k_pool + dst) = *reinterpret_cast<const uint4*>(k_new + src);
  *reinterpret_cast<uint4*>(v_pool + dst) = *reinterpret_cast<const uint4*>(v_new + src);
}

// One thread per (token, KV head, 4 consecutive elements): a 4-byte store of
// four key codes and one of four value codes into the slot's rows.  Four
// elements per thread keep enough waves in flight to hide the fp64 division
// of each element.  With block_tables non-null (a decode
// step, token n = row n) the thread of (n, head 0, elements 0..3) also moves
// the row forward, as append_step_kernel does.
template <bool I8>
__global__ __launch_bounds__(256) void append_codes_kernel(uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                         const float* __restrict__ scales,
                                                         const uint16_t* __restrict__ k_new,
                                                         const uint16_t* __restrict__ v_new,
                                                         const int32_t* __restrict__ slot_mapping, int num_tokens,
                                                         int hkv, int d, int block_size, int64_t num_slots,
                                                         int32_t* __restrict__ block_tables,
                                                         int32_t* __restrict__ context_lens, int max_blocks) {
  const int quads = d / 4;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int c4 = static_cast<int>(gid % quads);
  const int64_t th = gid / quads;
  const int j = static_cast<int>(th % hkv);
  const int64_t t = th / hkv;
  if (t >= num_tokens) return;
  const int64_t slot = slot_mapping[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t pb = slot / block_size;
  const int off = static_cast<int>(slot % block_size);
  if (block_tables != nullptr && j == 0 && c4 == 0) {
    const int pos = context_lens[t];
    if (pos >= 0 && pos / block_size < max_blocks && pos % block_size == off) {
      block_tables[t * max_blocks + pos / block_size] = static_cast<int32_t>(pb);
      context_lens[t] = pos + 1;
    }
  }
  const int64_t head = pb * hkv + j;
  const float2 kvs = *reinterpret_cast<const float2*>(scales + 2 * head);  // [num_blocks][Hkv][2]
  const float ks = kvs.x, vs = kvs.y;
  const int e0 = c4 * 4;  // first element
  const int64_t src = (t * hkv + j) * d + e0;
  const uint2 kin = *reinterpret_cast<const uint2*>(k_new + src);
  const uint2 vin = *reinterpret_cast<const uint2*>(v_new + src);
  const uint32_t kb[4] = {kin.x & 0xffffu, kin.x >> 16, kin.y & 0xffffu, kin.y >> 16};
  const uint32_t vb[4] = {vin.x & 0xffffu, vin.x >> 16, vin.y & 0xffffu, vin.y >> 16};
  uint32_t kw = 0, vw = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    kw |= code8<I8>(bf16_bits_to_f32(kb[e]), ks) << (8 * e);
    vw |= code8<I8>(bf16_bits_to_f32(vb[e]), vs) << (8 * e);
  }
  const int64_t dst = (head * block_size + off) * d + e0;
  *reinterpret_cast<uint32_t*>(k_pool + dst) = kw;
  *reinterpret_cast<uint32_t*>(v_pool + dst) = vw;
}

// grid = (ceil((2 * n16 + scales_per_block) / 256), num_pairs, num_layers);
// each thread moves 16 bytes of a block image, or one of the block's scales
// when the pools hold one-byte codes (scales [num_blocks][Hkv][2]:
// scales_per_block = 2 Hkv, else 0).
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_pool, uint8_t* __restrict__ v_pool,
                                                          const int32_t* __restrict__ pairs, int64_t block_bytes,
                                                          int num_blocks, int64_t layer_stride_bytes,
                                                          float* __restrict__ scales, int scales_per_block,
                                                          int64_t scale_layer_stride) {
  const int64_t n16 = block_bytes / 16;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= 2 * n16 + scales_per_block) return;
  const int32_t src = pairs[2 * blockIdx.y];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  if (idx >= 2 * n16) {
    const int64_t h = idx - 2 * n16;
    float* sc = scales + static_cast<int64_t>(blockIdx.z) * scale_layer_stride;
    sc[static_cast<int64_t>(dst) * scales_per_block + h] = sc[static_cast<int64_t>(src) * scales_per_block + h];
    return;
  }
  uint8_t* base = (idx < n16 ? k_pool : v_pool) + static_cast<int64_t>(blockIdx.z) * layer_stride_bytes;
  const int64_t i = idx < n16 ? idx : idx - n16;
  const uint4* s = reinterpret_cast<const uint4*>(base + src * block_bytes) + i;
  uint4* t = reinterpret_cast<uint4*>(base + dst * block_bytes) + i;
  *t = *s;
}

// Block images between two pools (preemption by swapping, "PagedAttention:
// Virtual Memory for the KV Cache", section 19): pair (src, dst) copies block
// src of the source pool to block dst of the destination pool, in every
// layer.  Either pool may be device memory or pinned host memory mapped for
// the device (then each 16-byte access crosses PCIe).
// grid = (ceil((2 * n16 + scales_per_block) / 256), num_pairs, num_layers).
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    uint8_t* __restrict__ dst_k, uint8_t* __restrict__ dst_v, const uint8_t* __restrict__ src_k,
    const uint8_t* __restrict__ src_v, const int32_t* __restrict__ pairs, int64_t block_bytes, int src_blocks,
    int dst_blocks, int64_t src_layer_bytes, int64_t dst_layer_bytes, float* __restrict__ dst_sc,
    const float* __restrict__ src_sc, int scales_per_block, int64_t src_scale_layer, int64_t dst_scale_layer) {
  const int64_t n16 = block_bytes / 16;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= 2 * n16 + scales_per_block) return;
  const int32_t src = pairs[2 * blockIdx.y];
  const int32_t dst = pairs[2 * blockIdx.y + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const int64_t layer = blockIdx.z;
  if (idx >= 2 * n16) {
    const int64_t h = idx - 2 * n16;
    const float* ss = src_sc + layer * src_scale_layer;
    float* ds = dst_sc + layer * dst_scale_layer;
    ds[static_cast<int64_t>(dst) * scales_per_block + h] = ss[static_cast<int64_t>(src) * scales_per_block + h];
    return;
  }
  const bool key = idx < n16;
  const int64_t i = key ? idx : idx - n16;
  const uint4* sp = reinterpret_cast<const uint4*>((key ? src_k : src_v) + layer * src_layer_bytes + src * block_bytes);
  uint4* dp = reinterpret_cast<uint4*>((key ? dst_k : dst_v) + layer * dst_layer_bytes + dst * block_bytes);
  dp[i] = sp[i];
}

bool shape_ok(int hkv, int d, int block_size, int dtype) {
  return hkv > 0 && (d == 64 || d == 128) && (block_size == 8 || block_size == 16 || block_size == 32) &&
         (dtype == PA_F32 || dtype == PA_BF16);
}

}  // namespace
}  // namespace pa

extern "C" int pa_append_kv(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                            const int32_t* slot_mapping, int num_tokens, int Hkv, int d_head,
                            int block_size, int num_blocks, int dtype, void* stream) {
  using namespace pa;
  if (num_tokens < 0 || num_blocks < 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (!shape_ok(Hkv, d_head, block_size, dtype)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  const int x = 16 / elem_bytes(dtype);
  const int64_t threads = static_cast<int64_t>(num_tokens) * Hkv * (d_head / x);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return PA_ERR_INVALID_ARG;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PA_BF16) {
    append_kv_kernel<uint16_t><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s>>>(
        static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), static_cast<const uint16_t*>(k_new),
        static_cast<const uint16_t*>(v_new), slot_mapping, num_tokens, Hkv, d_head, block_size, num_slots);
  } else {
    append_kv_kernel<float><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s>>>(
        static_cast<float*>(k_pool), static_cast<float*>(v_pool), static_cast<const float*>(k_new),
        static_cast<const float*>(v_new), slot_mapping, num_tokens, Hkv, d_head, block_size, num_slots);
  }
  return launch_status();
}

extern "C" int pa_append_step(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                              const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                              int num_seqs, int max_blocks_per_seq, int Hkv, int d_head, int block_size,
                              int num_blocks, int dtype, void* stream) {
  using namespace pa;
  if (num_seqs < 0 || num_blocks < 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (!shape_ok(Hkv, d_head, block_size, dtype)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (max_blocks_per_seq < 1) return PA_ERR_INVALID_ARG;
  if (!k_pool || !v_pool || !k_new || !v_new || !slot_mapping || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  const int x = 16 / elem_bytes(dtype);
  const int64_t threads = static_cast<int64_t>(num_seqs) * Hkv * (d_head / x);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return PA_ERR_INVALID_ARG;
  const int64_t num_slots = static_cast<int64_t>(num_blocks) * block_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == PA_BF16) {
    append_step_kernel<uint16_t><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s>>>(
        static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), static_cast<const uint16_t*>(k_new),
        static_cast<const uint16_t*>(v_new), slot_mapping, block_tables, context_lens, num_seqs,
        max_blocks_per_seq, Hkv, d_head, block_size, num_slots);
  } else {
    append_step_kernel<float><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, s>>>(
        static_cast<float*>(k_pool), static_cast<float*>(v_pool), static_cast<const float*>(k_new),
        static_cast<const float*>(v_new), slot_mapping, block_tables, context_lens, num_seqs,
        max_blocks_per_seq, Hkv, d_head, block_size, num_slots);
  }
  return launch_status();
}

extern "C" int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* src_dst_pairs, int num_pairs,
                              int Hkv, int d_head, int block_size, int num_blocks, int num_layers,
                              int64_t layer_stride_elems, int dtype, void* stream) {
  using namespace pa;
  if (num_pairs < 0 || num_blocks < 0 || num_layers <= 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if (!shape_ok(Hkv, d_head, block_size, dtype)) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !src_dst_pairs) return PA_ERR_INVALID_ARG;
  if (num_pairs > 65535 || num_layers > 65535) return PA_ERR_UNSUPPORTED;
  const int64_t eb = elem_bytes(dtype);
  const int64_t block_bytes = static_cast<int64_t>(Hkv) * d_head * block_size * eb;
  if (num_layers > 1 && layer_stride_elems < static_cast<int64_t>(num_blocks) * Hkv * d_head * block_size)
    return PA_ERR_INVALID_ARG;
  const int64_t layer_stride_bytes = num_layers > 1 ? layer_stride_elems * eb : 0;
  const int64_t gx = (2 * (block_bytes / 16) + 255) / 256;
  copy_blocks_kernel<<<dim3(static_cast<uint32_t>(gx), num_pairs, num_layers), dim3(256), 0,
                       static_cast<hipStream_t>(stream)>>>(static_cast<uint8_t*>(k_pool),
                                                          static_cast<uint8_t*>(v_pool), src_dst_pairs,
                                                          block_bytes, num_blocks, layer_stride_bytes, nullptr, 0,
                                                          0);
  return launch_status();
}

namespace pa {
namespace {

template <bool I8>
int append_codes(void* k_pool, void* v_pool, const float* scales, const void* k_new,
                 const void* v_new, const int32_t* slot_mapping, int num_tokens, int Hkv, int d_head, int block_size,
                 int num_blocks, void* stream) {
  if (num_tokens < 0 || num_blocks < 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  if (!shape_ok(Hkv, d_head, block_size, PA_BF16)) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!k_pool || !v_pool || !scales || !k_new || !v_new || !slot_mapping) return PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(scales) % 8 != 0) return PA_ERR_INVALID_ARG;
  const int64_t threads = static_cast<int64_t>(num_tokens) * Hkv * (d_head / 4);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return PA_ERR_INVALID_ARG;
  append_codes_kernel<I8><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), scales,
      static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slot_mapping, num_tokens, Hkv, d_head,
      block_size, static_cast<int64_t>(num_blocks) * block_size, nullptr, nullptr, 0);
  return launch_status();
}

template <bool I8>
int append_step_codes(void* k_pool, void* v_pool, const float* scales, const void* k_new,
                      const void* v_new, const int32_t* slot_mapping, int32_t* block_tables, int32_t* context_lens,
                      int num_seqs, int max_blocks_per_seq, int Hkv, int d_head, int block_size, int num_blocks,
                      void* stream) {
  if (num_seqs < 0 || num_blocks < 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
  if (!shape_ok(Hkv, d_head, block_size, PA_BF16)) return PA_ERR_UNSUPPORTED;
  if (num_seqs == 0) return PA_OK;
  if (max_blocks_per_seq < 1) return PA_ERR_INVALID_ARG;
  if (!k_pool || !v_pool || !scales || !k_new || !v_new || !slot_mapping || !block_tables || !context_lens)
    return PA_ERR_INVALID_ARG;
  if (reinterpret_cast<uintptr_t>(scales) % 8 != 0) return PA_ERR_INVALID_ARG;
  const int64_t threads = static_cast<int64_t>(num_seqs) * Hkv * (d_head / 4);
  const int64_t grid = (threads + 255) / 256;
  if (grid > INT32_MAX) return PA_ERR_INVALID_ARG;
  append_codes_kernel<I8><<<dim3(static_cast<uint32_t>(grid)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), scales,
      static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new), slot_mapping, num_seqs, Hkv, d_head,
      block_size, static_cast<int64_t>(num_blocks) * block_size, block_tables, context_lens, max_blocks_per_seq);
  return launch_status();
}

}  // namespace
}  // namespace pa

extern "C" int pa_append_kv_fp8(void* k_pool, void* v_pool, const float* scales,
                                const void* k_new, const void* v_new, const int32_t* slot_mapping, int num_tokens,
                                int Hkv, int d_head, int block_size, int num_blocks, void* stream) {
  return pa::append_codes<false>(k_pool, v_pool, scales, k_new, v_new, slot_mapping, num_tokens, Hkv,
                                 d_head, block_size, num_blocks, stream);
}

extern "C" int pa_append_kv_int8(void* k_pool, void* v_pool, const float* scales,
                                 const void* k_new, const void* v_new, const int32_t* slot_mapping, int num_tokens,
                                 int Hkv, int d_head, int block_size, int num_blocks, void* stream) {
  return pa::append_codes<true>(k_pool, v_pool, scales, k_new, v_new, slot_mapping, num_tokens, Hkv,
                                d_head, block_size, num_blocks, stream);
}

extern "C" int pa_append_step_fp8(void* k_pool, void* v_pool, const float* scales,
                                  const void* k_new, const void* v_new, const int32_t* slot_mapping,
                                  int32_t* block_tables, int32_t* context_lens, int num_seqs, int max_blocks_per_seq,
                                  int Hkv, int d_head, int block_size, int num_blocks, void* stream) {
  return pa::append_step_codes<false>(k_pool, v_pool, scales, k_new, v_new, slot_mapping, block_tables,
                                      context_lens, num_seqs, max_blocks_per_seq, Hkv, d_head, block_size, num_blocks,
                                      stream);
}

extern "C" int pa_append_step_int8(void* k_pool, void* v_pool, const float* scales,
                                   const void* k_new, const void* v_new, const int32_t* slot_mapping,
                                   int32_t* block_tables, int32_t* context_lens, int num_seqs, int max_blocks_per_seq,
                                   int Hkv, int d_head, int block_size, int num_blocks, void* stream) {
  return pa::append_step_codes<true>(k_pool, v_pool, scales, k_new, v_new, slot_mapping, block_tables,
                                     context_lens, num_seqs, max_blocks_per_seq, Hkv, d_head, block_size, num_blocks,
                                     stream);
}

extern "C" int pa_copy_blocks_fp8(void* k_pool, void* v_pool, float* scales,
                                  const int32_t* src_dst_pairs, int num_pairs, int Hkv, int d_head, int block_size,
                                  int num_blocks, int num_layers, int64_t layer_stride_elems,
                                  int64_t scale_layer_stride, void* stream) {
  using namespace pa;
  if (num_pairs < 0 || num_blocks < 0 || num_layers <= 0 || Hkv <= 0 || d_head <= 0 || block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (!shape_ok(Hkv, d_head, block_size, PA_BF16)) return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!k_pool || !v_pool || !scales || !src_dst_pairs) return PA_ERR_INVALID_ARG;
  if (num_pairs > 65535 || num_layers > 65535) return PA_ERR_UNSUPPORTED;
  const int64_t block_bytes = static_cast<int64_t>(Hkv) * d_head * block_size;
  if (num_layers > 1 && (layer_stride_elems < static_cast<int64_t>(num_blocks) * block_bytes ||
                         scale_layer_stride < static_cast<int64_t>(num_blocks) * Hkv * 2))
    return PA_ERR_INVALID_ARG;
  const int64_t gx = (2 * (block_bytes / 16) + 2 * Hkv + 255) / 256;  // images, then 2 Hkv scales
  copy_blocks_kernel<<<dim3(static_cast<uint32_t>(gx), num_pairs, num_layers), dim3(256), 0,
                       static_cast<hipStream_t>(stream)>>>(
      static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), src_dst_pairs, block_bytes, num_blocks,
      num_layers > 1 ? layer_stride_elems : 0, scales, 2 * Hkv, num_layers > 1 ? scale_layer_stride : 0);
  return launch_status();
}

namespace {
int swap_impl(void* dst_k, void* dst_v, const void* src_k, const void* src_v, const int32_t* pairs, int num_pairs,
              int Hkv, int d_head, int block_size, int elem, int src_blocks, int dst_blocks, int num_layers,
              int64_t src_layer_elems, int64_t dst_layer_elems, float* dst_sc, const float* src_sc,
              int64_t src_scale_layer, int64_t dst_scale_layer, void* stream) {
  using namespace pa;
  if (num_pairs < 0 || src_blocks < 0 || dst_blocks < 0 || num_layers <= 0 || Hkv <= 0 || d_head <= 0 ||
      block_size <= 0)
    return PA_ERR_INVALID_ARG;
  if (!(d_head == 64 || d_head == 128) || !(block_size == 8 || block_size == 16 || block_size == 32))
    return PA_ERR_UNSUPPORTED;
  if (num_pairs == 0) return PA_OK;
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs) return PA_ERR_INVALID_ARG;
  if (num_pairs > 65535 || num_layers > 65535) return PA_ERR_UNSUPPORTED;
  const int64_t block_elems = static_cast<int64_t>(Hkv) * d_head * block_size;
  const int64_t block_bytes = block_elems * elem;
  if (num_layers > 1 && (src_layer_elems < static_cast<int64_t>(src_blocks) * block_elems ||
                         dst_layer_elems < static_cast<int64_t>(dst_blocks) * block_elems))
    return PA_ERR_INVALID_ARG;
  const bool scales = src_sc != nullptr;
  const int spb = scales ? 2 * Hkv : 0;  // [num_blocks][Hkv][2]
  if (scales && num_layers > 1 &&
      (src_scale_layer < static_cast<int64_t>(src_blocks) * spb || dst_scale_layer < static_cast<int64_t>(dst_blocks) * spb))
    return PA_ERR_INVALID_ARG;
  const int64_t gx = (2 * (block_bytes / 16) + spb + 255) / 256;
  swap_blocks_kernel<<<dim3(static_cast<uint32_t>(gx), num_pairs, num_layers), dim3(256), 0,
                       static_cast<hipStream_t>(stream)>>>(
      static_cast<uint8_t*>(dst_k), static_cast<uint8_t*>(dst_v), static_cast<const uint8_t*>(src_k),
      static_cast<const uint8_t*>(src_v), pairs, block_bytes, src_blocks, dst_blocks,
      num_layers > 1 ? src_layer_elems * elem : 0, num_layers > 1 ? dst_layer_elems * elem : 0, dst_sc, src_sc, spb,
      num_layers > 1 ? src_scale_layer : 0, num_layers > 1 ? dst_scale_layer : 0);
  return launch_status();
}
}  // namespace

extern "C" int pa_swap_blocks(void* dst_k_pool, void* dst_v_pool, const void* src_k_pool, const void* src_v_pool,
                              const int32_t* src_dst_pairs, int num_pairs, int Hkv, int d_head, int block_size,
                              int dtype, int src_num_blocks, int dst_num_blocks, int num_layers,
                              int64_t src_layer_stride_elems, int64_t dst_layer_stride_elems, void* stream) {
  using namespace pa;
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  return swap_impl(dst_k_pool, dst_v_pool, src_k_pool, src_v_pool, src_dst_pairs, num_pairs, Hkv, d_head, block_size,
                   elem_bytes(dtype), src_num_blocks, dst_num_blocks, num_layers, src_layer_stride_elems,
                   dst_layer_stride_elems, nullptr, nullptr, 0, 0, stream);
}

extern "C" int pa_swap_blocks_fp8(void* dst_k_pool, void* dst_v_pool, float* dst_scales, const void* src_k_pool,
                                  const void* src_v_pool, const float* src_scales, const int32_t* src_dst_pairs, int num_pairs, int Hkv,
                                  int d_head, int block_size, int src_num_blocks, int dst_num_blocks, int num_layers,
                                  int64_t src_layer_stride_elems, int64_t dst_layer_stride_elems,
                                  int64_t src_scale_layer_stride, int64_t dst_scale_layer_stride, void* stream) {
  using namespace pa;
  if (num_pairs > 0 && (!dst_scales || !src_scales)) return PA_ERR_INVALID_ARG;
  return swap_impl(dst_k_pool, dst_v_pool, src_k_pool, src_v_pool, src_dst_pairs, num_pairs, Hkv, d_head, block_size,
                   1, src_num_blocks, dst_num_blocks, num_layers, src_layer_stride_elems, dst_layer_stride_elems,
                   dst_scales, src_scales, src_scale_layer_stride, dst_scale_layer_stride,
                   stream);
}

// An INT8 cache moves as an FP8 cache does: one-byte codes and their scales.
extern "C" int pa_copy_blocks_int8(void* k_pool, void* v_pool, float* scales,
                                   const int32_t* src_dst_pairs, int num_pairs, int Hkv, int d_head, int block_size,
                                   int num_blocks, int num_layers, int64_t layer_stride_elems,
                                   int64_t scale_layer_stride, void* stream) {
  return pa_copy_blocks_fp8(k_pool, v_pool, scales, src_dst_pairs, num_pairs, Hkv, d_head, block_size,
                            num_blocks, num_layers, layer_stride_elems, scale_layer_stride, stream);
}

extern "C" int pa_swap_blocks_int8(void* dst_k_pool, void* dst_v_pool, float* dst_scales, const void* src_k_pool,
                                   const void* src_v_pool, const float* src_scales, const int32_t* src_dst_pairs, int num_pairs, int Hkv,
                                   int d_head, int block_size, int src_num_blocks, int dst_num_blocks, int num_layers,
                                   int64_t src_layer_stride_elems, int64_t dst_layer_stride_elems,
                                   int64_t src_scale_layer_stride, int64_t dst_scale_layer_stride, void* stream) {
  return pa_swap_blocks_fp8(dst_k_pool, dst_v_pool, dst_scales, src_k_pool, src_v_pool, src_scales, src_dst_pairs, num_pairs, Hkv, d_head, block_size, src_num_blocks,
                            dst_num_blocks, num_layers, src_layer_stride_elems, dst_layer_stride_elems,
                            src_scale_layer_stride, dst_scale_layer_stride, stream);
}

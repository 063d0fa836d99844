// Validation of a decode batch on the device: the lengths and block-table
// entries the decode kernels would read, checked against the sizes the caller
// gives ("PagedAttention: Virtual Memory for the KV Cache", section 7: token i
// of a sequence lives in physical block block_table[i / B]; section 8: the
// table holds int32 ids of the pool's blocks).  The decode kernels never
// dereference an id outside the pool -- its tokens are left out -- and leave
// out tokens past max_blocks_per_seq * B; this call makes such inputs visible.
// The same for the copy-on-write pairs of a step (same page, sections 15-16: a
// copy clones a shared block into a fresh one): the block manager never names
// a destination twice or a destination that is also a source, and the copy
// kernel relies on that.

#include "common.h"

namespace pa {
namespace {

constexpr int kCheckThreads = 1024;

__device__ __forceinline__ int block_sum(int v, int* red) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) v += __shfl_xor(v, sh);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = 0;
  for (int w = 0; w < kCheckThreads / 64; ++w) t += red[w];
  return t;
}

__device__ __forceinline__ int block_min(int v, int* red) {
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) v = min(v, __shfl_xor(v, sh));
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  int t = INT32_MAX;
  for (int w = 0; w < kCheckThreads / 64; ++w) t = min(t, red[w]);
  return t;
}

// One workgroup: status[0] = rows whose length lies outside [0, max_ctx] or
// needs more than max_blocks table entries; status[1] = table entries (of the
// other rows, within their ceil(S / B) blocks) outside [0, num_blocks);
// status[2] = the first row of the first kind, status[3] = the first row
// holding one of the second (-1 when none).  Every word is written.
__global__ __launch_bounds__(kCheckThreads) void check_batch_kernel(const int32_t* __restrict__ block_tables,
                                                                   const int32_t* __restrict__ context_lens,
                                                                   int n_seqs, int max_blocks, int max_ctx,
                                                                   int num_blocks, int block_size,
                                                                   int32_t* __restrict__ status) {
  __shared__ int red[kCheckThreads / 64];
  int bad_rows = 0, bad_entries = 0;
  int first_row = INT32_MAX, first_entry_row = INT32_MAX;
  for (int n = threadIdx.x; n < n_seqs; n += kCheckThreads) {
    const int S = context_lens[n];
    const bool row_ok = S >= 0 && S <= max_ctx && (static_cast<int64_t>(S) + block_size - 1) / block_size <= max_blocks;
    if (!row_ok) {
      ++bad_rows;
      first_row = min(first_row, n);
    }
  }
  // entries: thread t walks entry t, t + 1024, ... of the flattened table
  const int64_t total = static_cast<int64_t>(n_seqs) * max_blocks;
  for (int64_t i = threadIdx.x; i < total; i += kCheckThreads) {
    const int n = static_cast<int>(i / max_blocks);
    const int lb = static_cast<int>(i - static_cast<int64_t>(n) * max_blocks);
    const int S = context_lens[n];
    if (S < 0 || S > max_ctx) continue;  // a bad row: counted above
    const int64_t need = (static_cast<int64_t>(S) + block_size - 1) / block_size;
    if (lb >= need) continue;
    const int e = block_tables[i];
    if (e < 0 || e >= num_blocks) {
      ++bad_entries;
      first_entry_row = min(first_entry_row, n);
    }
  }
  bad_rows = block_sum(bad_rows, red);
  bad_entries = block_sum(bad_entries, red);
  first_row = block_min(first_row, red);
  first_entry_row = block_min(first_entry_row, red);
  if (threadIdx.x == 0) {
    status[0] = bad_rows;
    status[1] = bad_entries;
    status[2] = first_row == INT32_MAX ? -1 : first_row;
    status[3] = first_entry_row == INT32_MAX ? -1 : first_entry_row;
  }
}

}  // namespace
}  // namespace pa

extern "C" int pa_check_batch(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                              int max_blocks_per_seq, int max_context_len, int num_blocks, int block_size,
                              int32_t* status, void* stream) {
  using namespace pa;
  if (num_seqs < 0 || max_blocks_per_seq < 1 || max_context_len < 0 || num_blocks < 0 || block_size < 1 || !status)
    return PA_ERR_INVALID_ARG;
  if (num_seqs > 0 && (!block_tables || !context_lens)) return PA_ERR_INVALID_ARG;
  check_batch_kernel<<<dim3(1), dim3(kCheckThreads), 0, static_cast<hipStream_t>(stream)>>>(
      block_tables, context_lens, num_seqs, max_blocks_per_seq, max_context_len, num_blocks, block_size, status);
  return launch_status();
}

namespace pa {
namespace {

constexpr int kPairThreads = 1024;
constexpr int kPairMaxBlocks = 1 << 19;        // two bitmaps of the pool: 2 x 64 KiB of LDS
constexpr int kPairWords = kPairMaxBlocks / 32;

// One workgroup over the pairs, with bitmaps of the pool's blocks in LDS.
// status: [0] pairs with an id outside [0, num_blocks) (the copy skips them),
// [1] pairs beyond the first that name an already named dst, [2] pairs whose
// dst is also some pair's src, [3] the lowest pair index counted in [0] or [2]
// or sharing its dst with another pair (-1 when none).  Each count depends only
// on the pairs, not on the order the threads run in.
__global__ __launch_bounds__(kPairThreads) void check_pairs_kernel(const int32_t* __restrict__ pairs, int n_pairs,
                                                                  int num_blocks, int32_t* __restrict__ status) {
  __shared__ uint32_t once[kPairWords], twice[kPairWords];
  __shared__ int red[kPairThreads / 64];
  const int words = (num_blocks + 31) / 32;
  const auto in_pool = [&](int s, int d) { return s >= 0 && s < num_blocks && d >= 0 && d < num_blocks; };
  int outside = 0, named = 0, distinct = 0, dst_src = 0, first = INT32_MAX;
  for (int w = threadIdx.x; w < words; w += kPairThreads) once[w] = twice[w] = 0;
  __syncthreads();
  // dsts named once, and twice or more
  for (int i = threadIdx.x; i < n_pairs; i += kPairThreads) {
    const int s = pairs[2 * i], d = pairs[2 * i + 1];
    if (!in_pool(s, d)) {
      ++outside;
      first = min(first, i);
      continue;
    }
    ++named;
    const uint32_t m = 1u << (d & 31);
    if (atomicOr(&once[d >> 5], m) & m) atomicOr(&twice[d >> 5], m);
  }
  __syncthreads();
  for (int w = threadIdx.x; w < words; w += kPairThreads) distinct += __popc(once[w]);
  for (int i = threadIdx.x; i < n_pairs; i += kPairThreads) {
    const int s = pairs[2 * i], d = pairs[2 * i + 1];
    if (in_pool(s, d) && (twice[d >> 5] & (1u << (d & 31)))) first = min(first, i);
  }
  __syncthreads();
  // srcs, then the dsts among them
  for (int w = threadIdx.x; w < words; w += kPairThreads) once[w] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n_pairs; i += kPairThreads) {
    const int s = pairs[2 * i], d = pairs[2 * i + 1];
    if (in_pool(s, d)) atomicOr(&once[s >> 5], 1u << (s & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < n_pairs; i += kPairThreads) {
    const int s = pairs[2 * i], d = pairs[2 * i + 1];
    if (in_pool(s, d) && (once[d >> 5] & (1u << (d & 31)))) {
      ++dst_src;
      first = min(first, i);
    }
  }
  outside = block_sum(outside, red);
  named = block_sum(named, red);
  distinct = block_sum(distinct, red);
  dst_src = block_sum(dst_src, red);
  first = block_min(first, red);
  if (threadIdx.x == 0) {
    status[0] = outside;
    status[1] = named - distinct;
    status[2] = dst_src;
    status[3] = first == INT32_MAX ? -1 : first;
  }
}

}  // namespace
}  // namespace pa

extern "C" int pa_check_pairs(const int32_t* src_dst_pairs, int num_pairs, int num_blocks, int32_t* status,
                              void* stream) {
  using namespace pa;
  if (num_pairs < 0 || num_blocks < 0 || !status) return PA_ERR_INVALID_ARG;
  if (num_pairs > 0 && !src_dst_pairs) return PA_ERR_INVALID_ARG;
  if (num_blocks > kPairMaxBlocks) return PA_ERR_UNSUPPORTED;
  check_pairs_kernel<<<dim3(1), dim3(kPairThreads), 0, static_cast<hipStream_t>(stream)>>>(src_dst_pairs, num_pairs,
                                                                                            num_blocks, status);
  return launch_status();
}

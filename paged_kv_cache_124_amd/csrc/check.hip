// Validation of a decode batch on the device: the lengths and block-table
// entries the decode kernels would read, checked against the sizes the caller
// gives ("PagedAttention: Virtual Memory for the KV Cache", section 7: token i
// of a sequence lives in physical block block_table[i / B]; section 8: the
// table holds int32 ids of the pool's blocks).  The decode kernels never
// dereference an id outside the pool -- its tokens are left out -- and leave
// out tokens past max_blocks_per_seq * B; this call makes such inputs visible.

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

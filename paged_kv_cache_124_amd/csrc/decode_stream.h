// Internal interface of the persistent decode kernel (decode_stream.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace pa {

struct StreamPlan {
  int workgroups = 0;          // persistent workgroups of 4 waves
  size_t prefix_offset = 0;    // workspace: [tile prefix sums | step slots | summary records]
  size_t slots_offset = 0;
  size_t records_offset = 0;
  size_t lens_offset = 0;       // code-cache step: the rows as the decode saw them, [num_seqs]
  size_t whole_offset = 0;      // code-cache step: records of whole segments, [num_seqs][Hkv][g]
  size_t seq_group_offset = 0;  // decode_shared: tile range and record row of each sequence
  size_t workspace_bytes = 0;
  size_t lds_bytes = 0;
};

// Element format of the cache the decode reads: bf16 values, or one-byte
// codes with per-(block, KV head) scales (FP8 E4M3 or INT8).
enum KvCodes { kKvBf16 = 0, kKvE4m3 = 1, kKvInt8 = 2 };

// The step's new tokens for pa_decode_step: k_new / v_new [N][Hkv][D] and
// their slots (device-readable).
struct StepInputs {
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
};

bool stream_eligible(int num_seqs, int g, int d, int block_size, int dtype);
// Shapes the FP8-cache kernel serves (bf16 queries and outputs).
bool stream_eligible_fp8(int num_seqs, int g, int d, int block_size);
// fp8: 64-token tiles over an FP8 cache instead of 32-token bf16 tiles.
StreamPlan stream_plan(int num_seqs, int hq, int hkv, int d, int block_size, int max_ctx, bool fp8 = false);
// codes != kKvBf16: the pools hold one-byte codes with per-(block, KV head)
// key and value scales, interleaved [num_blocks][Hkv][2].
int launch_stream(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v, const int32_t* bt,
                  const int32_t* cl, void* out, void* ws, int n, int hq, int hkv, int d, int block_size,
                  int max_blocks, int num_blocks, float scale_log2, const StepInputs* step,
                  const float* scales = nullptr, int codes = kKvBf16);

// The INT8-cache instances of the kernel (decode_stream_i8.hip); launch_stream
// calls it for codes == kKvInt8.
int launch_stream_int8(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v,
                       const int32_t* bt, const int32_t* cl, void* out, void* ws, int n, int hq, int hkv, int d,
                       int block_size, int max_blocks, int num_blocks, float scale_log2, const StepInputs* step,
                       const float* scales);

// Shared-prefix kernel (decode_shared.hip): groups of consecutive rows whose
// first P tokens lie in the same full blocks, int32 [num_groups][3] =
// (first row, rows, P), read on the device.
bool shared_eligible(int num_seqs, int num_groups, int g, int d, int block_size, int dtype);
StreamPlan shared_plan(int num_seqs, int num_groups, int hq, int hkv, int d, int block_size, int max_ctx);
int launch_shared(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v, const int32_t* bt,
                  const int32_t* cl, const int32_t* groups, int n_groups, void* out, void* ws, int n, int hq,
                  int hkv, int d, int block_size, int max_blocks, int num_blocks, float scale_log2,
                  const StepInputs* step);

}  // namespace pa

// Internal interface of the persistent bf16 decode kernel (decode_stream.hip).
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
  size_t workspace_bytes = 0;
  size_t lds_bytes = 0;
};

// The step's new tokens for pa_decode_step: k_new / v_new [N][Hkv][D] and
// their slots (device-readable).
struct StepInputs {
  const void* k_new;
  const void* v_new;
  const int32_t* slots;
};

bool stream_eligible(int num_seqs, int g, int d, int block_size, int dtype);
StreamPlan stream_plan(int num_seqs, int hq, int hkv, int d, int block_size, int max_ctx);
int launch_stream(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v, const int32_t* bt,
                  const int32_t* cl, void* out, void* ws, int n, int hq, int hkv, int d, int block_size,
                  int max_blocks, int num_blocks, float scale_log2, const StepInputs* step);

}  // namespace pa

// The persistent decode kernel of decode_stream_kernel.h over an INT8 cache
// (signed 8-bit codes with per-(block, KV head) scales), in a compilation unit
// of its own: with both one-byte code formats instantiated in one unit, the
// host compilation pass rejects the second (it resolves the stage copy of one
// format and not of the other).

#include "decode_stream_kernel.h"

namespace pa {

int launch_stream_int8(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v,
                       const int32_t* bt, const int32_t* cl, void* out, void* ws, int n, int hq, int hkv, int d,
                       int block_size, int max_blocks, int num_blocks, float scale_log2, const StepInputs* step,
                       const float* scales) {
#define PA_STREAM_CASE(DD, BB)                                                                                       \
  if (d == DD && block_size == BB) {                                                                                 \
    launch_stream_db<DD, BB, kKvInt8>(p, s, q, k, v, bt, cl, out, ws, n, hq, hkv, max_blocks, num_blocks, scale_log2, \
                                      step, scales);                                                                 \
    return launch_status();                                                                                          \
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

// Paged decode attention: the host side of the persistent decode kernel of
// decode_stream_kernel.h -- the launch plan (workgroups, workspace layout),
// the resident-workgroup query and the dispatch over head size, block size and
// cache format (bf16 and FP8 E4M3 here; INT8 in decode_stream_i8.hip).

#include <mutex>

#include "decode_stream_kernel.h"

namespace pa {
namespace {

size_t stream_lds(int n_seqs) { return (2 * static_cast<size_t>(n_seqs) + 1) * sizeof(int32_t); }

// CU count of the current device, cached per device.  Without a device
// (host-only use) the MI355X figure (256 CUs) is assumed.
int device_cus() {
  static int cus[16] = {};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) {
    (void)hipGetLastError();
    return 256;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (cus[dev] == 0) {
    int c = 0;
    cus[dev] = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && c > 0 ? c : 256;
    (void)hipGetLastError();
  }
  return cus[dev];
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
  StreamPlan p;
  // One workgroup (4 waves, one per SIMD) per CU: with two or more per CU the
  // oldest waves win the memory pipe and the split's completion times spread.
  int64_t wgs = device_cus();
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
  p.lens_offset = p.records_offset + static_cast<size_t>(waves) * 2 * g * (d + 4) * sizeof(float);
  p.whole_offset = p.lens_offset + (fp8 ? prefix_bytes : 0);
  // code caches: one more record per (row, KV head) for a decode step, whose
  // merge kernel adds the new token to every segment, whole ones included
  p.workspace_bytes = p.whole_offset + (fp8 ? static_cast<size_t>(num_seqs) * hkv * g * (d + 4) * sizeof(float) : 0);
  p.lds_bytes = stream_lds(num_seqs);
  return p;
}

int launch_stream(const StreamPlan& p, hipStream_t s, const void* q, const void* k, const void* v, const int32_t* bt,
                  const int32_t* cl, void* out, void* ws, int n, int hq, int hkv, int d, int block_size,
                  int max_blocks, int num_blocks, float scale_log2, const StepInputs* step, const float* scales,
                  int codes) {
  if (codes != kKvBf16 && !scales) return PA_ERR_UNSUPPORTED;
  if (codes == kKvInt8)
    return launch_stream_int8(p, s, q, k, v, bt, cl, out, ws, n, hq, hkv, d, block_size, max_blocks, num_blocks,
                              scale_log2, step, scales);
#define PA_STREAM_CASE(DD, BB)                                                                                       \
  if (d == DD && block_size == BB) {                                                                                 \
    if (codes == kKvE4m3)                                                                                            \
      launch_stream_db<DD, BB, kKvE4m3>(p, s, q, k, v, bt, cl, out, ws, n, hq, hkv, max_blocks, num_blocks,          \
                                        scale_log2, step, scales);                                                   \
    else                                                                                                             \
      launch_stream_db<DD, BB, kKvBf16>(p, s, q, k, v, bt, cl, out, ws, n, hq, hkv, max_blocks, num_blocks,          \
                                        scale_log2, step, nullptr);                                                  \
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

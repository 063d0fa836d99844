// Internal helpers shared by the device entry points of libpa.so (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "pa.h"

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Partial-result precision of the split decode and the LDS/merge format use
// base-2 exponent arithmetic: scores are kept as s * log2(e) so that every
// exponential is one v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 b = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, b);
}

template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int kBytes = 4;
  __device__ static float load(const float* p) { return *p; }
  __device__ static void store(float* p, float v) { *p = v; }
};
template <>
struct Elem<uint16_t> {  // bf16 storage
  static constexpr int kBytes = 2;
  __device__ static float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  __device__ static void store(uint16_t* p, float v) { *p = f32_to_bf16_bits(v); }
};

// Cache policy of the loads that stream the KV pool: the non-temporal bit of
// the gfx9 cache-policy field (the "nt" modifier).  A decode reads each KV byte
// once per launch, and a launch reads far more than the L2 and the Infinity
// Cache hold, so keeping those lines buys nothing; loads marked non-temporal
// read a 4 GiB buffer about 11 % faster than default-policy loads on MI355X
// (7.1 against 6.4 TB/s, 16-byte loads, four 4 KiB pieces in flight per wave).
constexpr int kKvLoadPolicy = 2;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One 16-byte load of KV data with the streaming policy above.
__device__ __forceinline__ uint4 load_kv16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

inline int elem_bytes(int dtype) { return dtype == PA_F32 ? 4 : (dtype == PA_BF16 ? 2 : 0); }

inline int launch_status() {
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace pa

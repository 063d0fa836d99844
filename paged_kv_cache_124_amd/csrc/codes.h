// Quantizers of the one-byte KV caches, shared by the appends (kv_ops.hip)
// and the merge kernel of a decode step over such a cache, which attends to
// the new token before storing it (decode_stream_kernel.h): both must give
// the same code for the same value and scale.
#pragma once

#include "common.h"

namespace pa {
namespace {

// ---- FP8 (E4M3) cache ----------------------------------------------------------
//
// A value x goes into the cache under scale s as the sign of x and the finite
// E4M3 magnitude nearest to the real quotient |x| / s, ties to an even
// mantissa, saturating at 448 (E4M3 of the OCP 8-bit floating point format:
// exponent bias 7, subnormals, NaN at 0x7F / 0xFF).  The quotient is formed in
// fp64: for 24-bit x and s it is never rounded across a midpoint the exact
// quotient does not reach, so the code is the one the exact quotient gives.
// NaN input, or a scale that is not positive and finite, stores 0x7F.
// The code in two parts: e4m3_quotient forms y = |x| / s in fp64 (0 for bad
// input), e4m3_encode rounds it; a kernel forming several codes computes all
// quotients first, so that their divisions overlap.
__device__ __forceinline__ bool code_input_bad(float x, float s) { return !(s > 0.f) || !(s < INFINITY) || x != x; }

__device__ __forceinline__ double e4m3_quotient(float x, float s) {
  const double q = fabs(static_cast<double>(x)) / static_cast<double>(s);
  return code_input_bad(x, s) ? 0.0 : q;
}

__device__ __forceinline__ uint32_t e4m3_encode(double y, float x, float s) {
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  // No branch on the range: both candidates are formed and one is selected (as
  // is 0x7F for bad input).  Each candidate is computed from y clamped into its
  // own range, which changes only the candidate that is not selected; the
  // normal candidate's clamp at 448 is itself the saturation.
  // subnormal grid 2^-9 (code = multiple of 2^-9); 8 * 2^-9 is the smallest normal, code 0x08
  const uint32_t mag_sub = static_cast<uint32_t>(rint(fmin(y, 0x1p-6) * 512.0));
  const double yn = fmin(fmax(y, 0x1p-6), 448.0);
  int e2 = 0;
  (void)frexp(yn, &e2);                                 // yn = f * 2^e2, f in [0.5, 1)
  const int e = e2 - 1;                                 // floor(log2 yn), -6 .. 8
  const double m = rint(ldexp(yn, 3 - e));              // 8 .. 16 steps of 2^(e-3), ties to even
  // m = 16 carries into exponent e + 1; yn = 448 (every y >= 448 saturates) gives 0x7E
  const uint32_t mag_norm = static_cast<uint32_t>((e + 7) * 8) + static_cast<uint32_t>(m) - 8u;
  const uint32_t mag = y < 0x1p-6 ? mag_sub : mag_norm;
  return code_input_bad(x, s) ? 0x7Fu : sign | mag;
}

__device__ __forceinline__ uint32_t e4m3_code(float x, float s) { return e4m3_encode(e4m3_quotient(x, s), x, s); }

// INT8 cache: x goes in under scale s as the integer nearest to the real
// quotient x / s, ties to even, clamped to -127..127 (symmetric: negating x
// negates the code), two's complement.  The quotient is formed in fp64, exact
// for the decision by the argument above (a half-integer quotient of 24-bit x
// and s is exact; any other lies far from every half-integer).  An 8-bit
// integer has no NaN: NaN input, or a scale that is not positive and finite,
// stores 0.
__device__ __forceinline__ double i8_quotient(float x, float s) {
  const double q = static_cast<double>(x) / static_cast<double>(s);
  return code_input_bad(x, s) ? 0.0 : q;
}

__device__ __forceinline__ uint32_t i8_encode(double y, float x, float s) {
  const double c = y >= 127.0 ? 127.0 : (y <= -127.0 ? -127.0 : rint(y));  // rint: nearest, ties to even
  return code_input_bad(x, s) ? 0u : static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xFFu;
}

__device__ __forceinline__ uint32_t i8_code(float x, float s) { return i8_encode(i8_quotient(x, s), x, s); }

// The number a code stands for (before its scale): E4M3 sign, 4-bit exponent
// (bias 7; 0 = subnormal, steps of 2^-9) and 3-bit mantissa, NaN at 0x7F /
// 0xFF; INT8 the two's complement integer.  Exact in fp32.
template <bool I8>
__device__ __forceinline__ float code8_value(uint32_t c) {
  if constexpr (I8) {
    return static_cast<float>(static_cast<int8_t>(c & 0xFFu));
  } else {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    // normal: (1 + m / 8) * 2^(e - 7), built as fp32 bits; subnormal: m * 2^-9
    // (all selects, no branch)
    const float nrm = __uint_as_float(((e + 120u) << 23) | (m << 20));
    const float sub = static_cast<float>(m) * 0x1p-9f;
    const float mag = e == 15u && m == 7u ? __uint_as_float(0x7FC00000u) : (e == 0u ? sub : nrm);
    return (c & 0x80u) ? -mag : mag;
  }
}

template <bool I8>
__device__ __forceinline__ uint32_t code8(float x, float s) {
  if constexpr (I8)
    return i8_code(x, s);
  else
    return e4m3_code(x, s);
}

template <bool I8>
__device__ __forceinline__ double code8_quotient(float x, float s) {
  if constexpr (I8)
    return i8_quotient(x, s);
  else
    return e4m3_quotient(x, s);
}

template <bool I8>
__device__ __forceinline__ uint32_t code8_encode(double y, float x, float s) {
  if constexpr (I8)
    return i8_encode(y, x, s);
  else
    return e4m3_encode(y, x, s);
}

}  // namespace
}  // namespace pa

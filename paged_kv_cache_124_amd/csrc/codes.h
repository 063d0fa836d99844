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
__device__ __forceinline__ uint32_t e4m3_code(float x, float s) {
  if (!(s > 0.f) || !(s < INFINITY) || x != x) return 0x7Fu;
  const uint32_t sign = (__float_as_uint(x) >> 24) & 0x80u;
  const double y = fabs(static_cast<double>(x)) / static_cast<double>(s);
  uint32_t mag;
  if (y >= 448.0) {
    mag = 0x7Eu;
  } else if (y < 0x1p-6) {
    // subnormal grid 2^-9 (code = multiple of 2^-9); 8 * 2^-9 is the smallest normal, code 0x08
    mag = static_cast<uint32_t>(rint(y * 512.0));
  } else {
    int e2 = 0;
    (void)frexp(y, &e2);                                  // y = f * 2^e2, f in [0.5, 1)
    const int e = e2 - 1;                                 // floor(log2 y), -6 .. 8
    const double m = rint(ldexp(y, 3 - e));               // 8 .. 16 steps of 2^(e-3), ties to even
    mag = static_cast<uint32_t>((e + 7) * 8) + static_cast<uint32_t>(m) - 8u;  // m = 16 carries into e + 1
  }
  return sign | mag;
}

// INT8 cache: x goes in under scale s as the integer nearest to the real
// quotient x / s, ties to even, clamped to -127..127 (symmetric: negating x
// negates the code), two's complement.  The quotient is formed in fp64, exact
// for the decision by the argument above (a half-integer quotient of 24-bit x
// and s is exact; any other lies far from every half-integer).  An 8-bit
// integer has no NaN: NaN input, or a scale that is not positive and finite,
// stores 0.
__device__ __forceinline__ uint32_t i8_code(float x, float s) {
  if (!(s > 0.f) || !(s < INFINITY) || x != x) return 0u;
  const double y = static_cast<double>(x) / static_cast<double>(s);
  const double c = y >= 127.0 ? 127.0 : (y <= -127.0 ? -127.0 : rint(y));  // rint: nearest, ties to even
  return static_cast<uint32_t>(static_cast<int32_t>(c)) & 0xFFu;
}

// The number a code stands for (before its scale): E4M3 sign, 4-bit exponent
// (bias 7; 0 = subnormal, steps of 2^-9) and 3-bit mantissa, NaN at 0x7F /
// 0xFF; INT8 the two's complement integer.  Exact in fp32.
template <bool I8>
__device__ __forceinline__ float code8_value(uint32_t c) {
  if constexpr (I8) {
    return static_cast<float>(static_cast<int8_t>(c & 0xFFu));
  } else {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    const float mag = e == 15u && m == 7u ? NAN : (e == 0u ? ldexpf(static_cast<float>(m), -9)
                                                           : ldexpf(static_cast<float>(8u + m), static_cast<int>(e) - 10));
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

}  // namespace
}  // namespace pa

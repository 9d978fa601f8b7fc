// Device-side FP8 row encoding shared by the cache writes (pkv_fp8.hip) and
// the decode step that writes inside the 8-bit attention launch
// (pkv_kernels.hip), so both produce the same bits: E4M3 codes (OCP, round
// to nearest even, a zero code stored as +0) of x * 2^-e with e the smallest
// integer such that max|x| <= 448 * 2^e (clamped to [-126, 127]), the
// maximum taken over the row's finite elements; a non-finite element (an
// infinity or a NaN) is stored as the E4M3 NaN code with its sign.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace pkv {

// |x| for a finite x, 0 for an infinity or a NaN: the magnitude a row's
// scale is chosen from.
__device__ __forceinline__ float finite_abs(float x) {
  const float a = fabsf(x);
  return a <= 3.4028235e38f ? a : 0.f;          // false for +inf and NaN
}

// E4M3 byte of y: for a finite y with |y| <= 448 the nearest code, ties to
// an even mantissa; for an infinity or a NaN the NaN code S.1111.111.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a <= 3.4028235e38f)) return sign | 0x7fu;
  uint32_t c;
  if (a < 0x1p-6f) {
    c = static_cast<uint32_t>(rintf(a * 512.0f));                 // subnormal: m * 2^-9, m = 0..8
  } else {
    const int E = static_cast<int>((__float_as_uint(a) >> 23) & 0xffu) - 127;
    const float r = rintf(__builtin_amdgcn_ldexpf(a, 3 - E));      // 8 .. 16
    c = static_cast<uint32_t>(((E + 7) << 3) + static_cast<int>(r) - 8);
  }
  return c == 0 ? 0u : (sign | c);
}

// e of the row scale 2^e for a row whose largest magnitude is amax (>= 0).
__device__ __forceinline__ int row_exponent(float amax) {
  const uint32_t ab = __float_as_uint(amax);
  if (ab == 0) return 0;
  int E;
  uint32_t man;
  const uint32_t ef = ab >> 23;
  if (ef == 0) {                                  // float32 subnormal
    const int lz = __clz(ab);
    E = (31 - lz) - 149;
    man = (ab << (lz - 8)) & 0x7fffffu;
  } else {
    E = static_cast<int>(ef) - 127;
    man = ab & 0x7fffffu;
  }
  const int e = E - 8 + (man > 0x600000u ? 1 : 0);  // 448 = 1.75 * 2^8
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}

}  // namespace pkv

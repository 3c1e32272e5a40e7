// Device helpers shared by the append and decode kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// E4M3 (OCP e4m3fn) code of y: nearest representable value, ties to the
// even code, finite magnitudes from 448 up saturate to +-448, NaN -> 0x7f.
// Below 2^-6 the grid is m * 2^-9 (rint of y * 512, exact scaling); above,
// the fp32 fraction is cut to 3 bits with round-to-nearest-even, a carry
// moving into the exponent as it should.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  if (!(a == a)) return 0x7fu;
  if (a >= 448.0f) return sign | 0x7eu;
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.0f);
  const uint32_t ua = __float_as_uint(a);
  uint32_t code = ((((ua >> 23) & 0xffu) - 127u + 7u) << 3) | ((ua >> 20) & 7u);
  const uint32_t rest = ua & 0xfffffu;  // the 20 fraction bits dropped
  if (rest > 0x80000u || (rest == 0x80000u && (code & 1u))) code += 1u;
  return sign | code;
}

// 16-bit element (binary16 when DT == 0, bfloat16 when DT == 1) as fp32.
template <int DT>
__device__ __forceinline__ float elem_to_float(uint32_t bits16) {
  if constexpr (DT == 1) return __uint_as_float(bits16 << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

}  // namespace pa

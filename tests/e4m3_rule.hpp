// Test-only: OCP FP8 E4M3 ("fn") encoder, the encoding rule of the fp8 cache
// write written out in C on integer bits.  The device takes the same rule
// with the hardware conversion (cache_write.hip, e4m3x2); this independent
// statement is compiled only into the CPU test library, where it is checked
// against the oracle's encoder.
#pragma once

#include <cmath>
#include <cstdint>
#include <cstring>

namespace kvc {

// Nearest E4M3 code of a float32 (ties to the even code), saturating at
// +-448; NaN gives 0x7F with the sign kept.  E4M3: 1 sign, 4 exponent bits
// (bias 7), 3 mantissa bits, subnormal spacing 2^-9, largest finite 448.
inline uint8_t e4m3_from_float(float y) {
  uint32_t bits;
  std::memcpy(&bits, &y, sizeof(bits));
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t mag = bits & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return static_cast<uint8_t>(sign | 0x7Fu);   // NaN
  if (mag >= 0x43E00000u) return static_cast<uint8_t>(sign | 0x7Eu);  // |y| >= 448
  if (mag < 0x3C800000u) {
    // |y| < 2^-6: multiples of 2^-9; the scaling by 2^9 is exact and rintf
    // rounds half to even.  A result of 8 is the smallest normal, code 0x08.
    const float a = std::fabs(y) * 512.0f;
    return static_cast<uint8_t>(sign | static_cast<uint32_t>(rintf(a)));
  }
  // Normal range: keep 3 of the 23 mantissa bits, round to nearest even on
  // the 20 dropped bits (a carry moves into the exponent), then rebias the
  // exponent from 127 to 7.
  uint32_t r = mag + 0x7FFFFu + ((mag >> 20) & 1u);
  r >>= 20;
  uint32_t code = r - (120u << 3);
  if (code > 0x7Eu) code = 0x7Eu;
  return static_cast<uint8_t>(sign | code);
}

}  // namespace kvc

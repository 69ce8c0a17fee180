// float32 -> OCP FP8 E4M3FN code, the encoder of the FP8 KV-cache write
// (pd_rope.hip). Kept in a header of its own so that the same source also
// builds for the host, where a CPU test compares it with a nearest-code
// search written from the format's definition.
//
// The format (OCP 8-bit floating point, E4M3FN): 1 sign bit, 4 exponent
// bits with bias 7 and 3 fraction bits; exponent field 0 holds the
// subnormals f/8 * 2^-6; 0x7F and 0xFF are NaN, so the largest finite
// magnitude is 448 (0x7E). Encoding: the nearest value, ties to the even
// code; magnitudes from 464 up (whose nearest would be the NaN code) are
// held at 448; NaN gives 0x7F with the input's sign bit.
//
// PD_FP8_FN gives the function's qualifiers: the device build defines it as
// a device inline function before including this header; a host build gets
// a plain inline function.
#pragma once

#include <math.h>
#include <stdint.h>

#ifndef PD_FP8_FN
#define PD_FP8_FN inline
#endif

// Both ranges are computed and one kept by selects, so no lane branches.
PD_FP8_FN uint32_t e4m3_code(float f) {
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  // below 2^-6: steps of 2^-9, codes 0 .. 8 (the input clamped so that the
  // conversion stays in range where this result is not kept)
  const uint32_t sub =
      (uint32_t)__builtin_rintf(fminf(__builtin_bit_cast(float, a), 0.015625f) * 512.0f);
  // from 2^-6: keep 3 of the 23 fraction bits (nearest-even), rebias 127 -> 7
  const uint32_t nrm = ((a + 0x7ffffu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  uint32_t c = a < 0x3c800000u ? sub : nrm;
  c = a >= 0x43e80000u ? 0x7eu : c;
  c = a > 0x7f800000u ? 0x7fu : c;
  return sign | c;
}

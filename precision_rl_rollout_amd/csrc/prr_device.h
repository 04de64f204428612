// Device-side helpers shared by the kernels of libprr (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prr {

constexpr int kBlock = 128;          // weight block edge, activation group
constexpr float kFp8Max = 448.0f;    // largest finite e4m3 magnitude
constexpr float kInt8Max = 127.0f;

// bf16 halves of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Running max of |x| over a word of two bf16 values, on bit patterns: for
// non-negative IEEE values the bit-pattern order is the value order, so a
// max over the 15-bit magnitudes of both halves gives amax exactly.
__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t m, uint32_t w) {
  const uint32_t a = w & 0x7FFF7FFFu;
  const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
  m = max(m, lo);
  return max(m, hi);
}

// Max over all 64 lanes of a wave (result in every lane).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 64));
  return v;
}

// Max over each aligned group of 16 lanes (result in every lane of it).
__device__ __forceinline__ uint32_t lane16_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, 16));
  return v;
}

// fl32(x / s), IEEE binary32 division with round-to-nearest-even.  HIP's
// fp32 '/' is correctly rounded by default (no fast-math flags are used
// anywhere in this library) and fp32 subnormals are preserved.
__device__ __forceinline__ float div_rn(float x, float s) { return x / s; }

// Saturating round-to-nearest-even OCP e4m3 code of an fp32 value, built
// from the fp32 fields with integer arithmetic (no conversion instruction):
//   |v| >= 448            -> 0x7E (saturate; NaN is never produced)
//   2^-6 <= |v| < 448     -> round the 23-bit mantissa to 3 bits, ties to
//                            even (add 0x7FFFF plus the kept LSB), then
//                            rebias the exponent from 127 to 7
//   |v| < 2^-6            -> subnormal: RNE(|v| * 2^9), exact scaling;
//                            a result of 8 is the smallest normal's code
// and the sign bit is copied (so -0 -> 0x80).
__device__ __forceinline__ uint32_t e4m3_code(float v) {
  const uint32_t b = __float_as_uint(v);
  const uint32_t a = b & 0x7FFFFFFFu;
  const uint32_t rn = a + 0x7FFFFu + ((a >> 20) & 1u);
  const uint32_t cn = (rn >> 20) - (120u << 3);
  const uint32_t cs = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
  uint32_t c = (a < 0x3C800000u) ? cs : cn;     // 0x3C800000 = 2^-6
  c = (a >= 0x43E00000u) ? 0x7Eu : c;           // 0x43E00000 = 448
  return c | ((b >> 24) & 0x80u);
}

// Four e4m3 codes packed little-endian into one word.
__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// Eight bf16 values (one 16-byte chunk) -> eight e4m3 codes (8 bytes).
// s == 0 only for an all-zero block, where every x is a signed zero and the
// code is its sign.
__device__ __forceinline__ uint2 e4m3_chunk(uint4 w, float s) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t word = ws[2 * h + j];
      const float x0 = bf16_lo(word), x1 = bf16_hi(word);
      const float v0 = (s != 0.0f) ? div_rn(x0, s) : x0;
      const float v1 = (s != 0.0f) ? div_rn(x1, s) : x1;
      c[2 * j] = e4m3_code(v0);
      c[2 * j + 1] = e4m3_code(v1);
    }
    out[h] = pack4(c[0], c[1], c[2], c[3]);
  }
  return make_uint2(out[0], out[1]);
}

// clamp(RNE(v), -127, 127) as a byte.
__device__ __forceinline__ uint32_t int8_code(float v) {
  float r = __builtin_rintf(v);
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (uint32_t)((int32_t)r) & 0xFFu;
}

__device__ __forceinline__ uint2 int8_chunk(uint4 w, float s) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t c[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const uint32_t word = ws[2 * h + j];
      const float x0 = bf16_lo(word), x1 = bf16_hi(word);
      c[2 * j] = (s != 0.0f) ? int8_code(div_rn(x0, s)) : 0u;
      c[2 * j + 1] = (s != 0.0f) ? int8_code(div_rn(x1, s)) : 0u;
    }
    out[h] = pack4(c[0], c[1], c[2], c[3]);
  }
  return make_uint2(out[0], out[1]);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

}  // namespace prr

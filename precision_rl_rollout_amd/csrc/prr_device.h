// Device-side helpers shared by the kernels of libprr (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prr {

// 16-byte load of data read exactly once (quantizer inputs): marked
// non-temporal so it streams past the caches instead of displacing lines.
__device__ __forceinline__ uint4 load_once16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t[0], t[1], t[2], t[3]);
}

constexpr int kBlock = 128;          // weight block edge, activation group
constexpr float kFp8Max = 448.0f;    // largest finite e4m3 magnitude
constexpr float kInt8Max = 127.0f;

// bf16 halves of a 32-bit word -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Running max of |x| over a word of two bf16 values, on bit patterns: for
// non-negative IEEE values the bit-pattern order is the value order, so a
// max over the 15-bit magnitudes of both halves gives amax exactly.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Packed form: keeps the two running maxima in the two halves of `m`
// (one v_pk_max_u16 per word); fold with absmax_fold() at the end.
__device__ __forceinline__ uint32_t absmax_bf16x2(uint32_t m, uint32_t w) {
  const u16x2 a = __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu);
  const u16x2 b = __builtin_bit_cast(u16x2, m);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ uint32_t absmax_fold(uint32_t m) { return max(m & 0xFFFFu, m >> 16); }

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
// anywhere in this library) and fp32 subnormals are preserved.  Used once
// per block, for the scale itself and the reciprocal below.
__device__ __forceinline__ float div_rn(float x, float s) { return x / s; }

// Division of every element of a block by the block's scale s > 0.
//
// A correctly rounded divide costs about ten VALU instructions; a block
// divides many elements by one s, so the reciprocal r = RN(1/s) is formed
// once and each quotient takes Markstein's correction step (P. Markstein,
// "Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Dev. 34(1), 1990; also Muller et al., "Handbook
// of Floating-Point Arithmetic", on division with an FMA):
//     y = RN(x r),  e = fma(-y, s, x)  (exact),  q = RN(e r + y).
// Blocks with s < 2^-64 first scale s and x by 2^96 (exact: both are
// powers-of-two multiples, and |x| <= 448 s stays tiny) so that the
// remainder never underflows where it matters.  The fma loses the sign of
// a zero quotient, which the copysign restores (x / s has the sign of x).
//
// Used only where its result is encoded to e4m3 or int8, and only with
// |x| <= 448 s (block scales; the KV-cache path clamps, below).  The GPU
// parity tests compare the encoded results with the oracle's
// encode(fl32(x / s)) byte for byte, through the library's quantizers, for
// every finite bf16 x with |x| <= amax (both signs) and s = fl32(amax / 448)
// or fl32(amax / 127), over 1,031 amax values spanning every bf16 binade:
// the power of two, 448 * 2^k (exact quotients, e4m3 ties), the largest
// and a random mantissa of each, and 16 subnormal amax values, so both the
// ordinary and the 2^96 path.  (By Markstein's theorem the step returns
// the correctly rounded quotient whenever its remainder e is exact; e can
// be inexact only for |x| below about 2^-100, near the fp32 subnormal
// range, and with s >= 2^-64 -- the 2^96 prescaling sees to it -- those
// quotients lie below 2^-36, far under the smallest nonzero e4m3 value
// 2^-9 or the int8 rounding point 1/2, and encode to zero either way.)
struct BlockDiv {
  float s;   // s, or s * 2^96
  float r;   // RN(1 / s) of the above
  bool tiny;
};

__device__ __forceinline__ BlockDiv block_div(float s) {
  BlockDiv d;
  d.tiny = s < 0x1p-64f;
  d.s = d.tiny ? s * 0x1p96f : s;
  d.r = div_rn(1.0f, d.s);
  return d;
}

template <bool kTiny>
__device__ __forceinline__ float div_block(float x, const BlockDiv& d) {
  if constexpr (kTiny) x *= 0x1p96f;
  const float y = x * d.r;
  const float e = __builtin_fmaf(-y, d.s, x);
  return __builtin_copysignf(__builtin_fmaf(e, d.r, y), x);
}

// Four e4m3 codes of four quotients, packed little-endian, by the hardware
// conversion (round to nearest even from the MODE register, e4m3 with
// subnormals).  It does not saturate: magnitudes in (464, 480] would give
// NaN.  Quotients of a block never exceed 448 * (1 + 2^-8) < 464 (the
// scale is amax / 448 rounded to fp32, relative error below 2^-8 even for
// subnormal scales), so no clamp is needed.  What the GPU parity tests
// check of it against the oracle's bit-built saturating RNE encoder: every
// quotient the sweep above produces, and every finite bf16 value itself
// (a KV-cache write with s = 1, whose quotients are exact).
__device__ __forceinline__ uint32_t cvt_e4m3x4(float q0, float q1, float q2, float q3) {
  int d = __builtin_amdgcn_cvt_pk_fp8_f32(q0, q1, 0, false);
  d = __builtin_amdgcn_cvt_pk_fp8_f32(q2, q3, d, true);
  return (uint32_t)d;
}

// Quotient saturated to +-448 (sign of zero kept): the saturating RNE code
// is unchanged, and the conversion then never sees |v| > 464.  Needed where
// a scale does not bound the quotients (a KV-cache scale calibrated on an
// earlier batch); block scales do bound them.  With such a scale x / s can
// exceed the binary32 range, and the correction step above then yields an
// infinity or a NaN (x r overflows, e = fma(-inf, s, x) = -inf, and
// fma(-inf, r, inf) is NaN); div_block gives it the sign of x, and every
// value that is not within [-448, 448] -- NaN included, as the comparison
// fails -- becomes 448 with its sign: the saturating code of a quotient
// beyond the range.
__device__ __forceinline__ float clamp448(float v) {
  return __builtin_fabsf(v) <= 448.0f ? v : __builtin_copysignf(448.0f, v);
}

// Eight bf16 values (one 16-byte chunk) -> eight e4m3 codes (8 bytes).
template <bool kTiny, bool kClamp = false>
__device__ __forceinline__ uint2 e4m3_chunk(uint4 w, const BlockDiv& d) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w0 = ws[2 * h], w1 = ws[2 * h + 1];
    float q[4] = {div_block<kTiny>(bf16_lo(w0), d), div_block<kTiny>(bf16_hi(w0), d),
                  div_block<kTiny>(bf16_lo(w1), d), div_block<kTiny>(bf16_hi(w1), d)};
    if constexpr (kClamp) {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = clamp448(q[e]);
    }
    out[h] = cvt_e4m3x4(q[0], q[1], q[2], q[3]);
  }
  return make_uint2(out[0], out[1]);
}

// An all-zero block (s == 0): every element is a signed zero and its code
// is its sign bit.
__device__ __forceinline__ uint2 e4m3_zero_chunk(uint4 w) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w0 = ws[2 * h], w1 = ws[2 * h + 1];
    out[h] = ((w0 >> 8) & 0x80u) | ((w0 >> 16) & 0x8000u) | ((w1 << 8) & 0x800000u) |
             (w1 & 0x80000000u);
  }
  return make_uint2(out[0], out[1]);
}

// e4m3 chunk for any block: dispatch on the block-uniform scale class.
template <bool kClamp = false>
__device__ __forceinline__ uint2 e4m3_chunk_any(uint4 w, float s, const BlockDiv& d) {
  if (s == 0.0f) return e4m3_zero_chunk(w);
  return d.tiny ? e4m3_chunk<true, kClamp>(w, d) : e4m3_chunk<false, kClamp>(w, d);
}

// Eight code bytes to an 8-byte aligned address.  kStream marks the store
// non-temporal: the L2 does not keep the line, which pays where the codes
// of a whole layer stack (more than the 256 MB last-level cache) are
// written back to back -- the one-launch stack re-quantization ran 6%
// faster with it -- and costs where one weight's codes are read again soon
// (7% slower on a 136 MB weight re-quantized in place).
template <bool kStream>
__device__ __forceinline__ void store_codes8(uint8_t* p, uint2 c) {
  if constexpr (kStream) {
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    __builtin_nontemporal_store(u32x2{c.x, c.y}, reinterpret_cast<u32x2*>(p));
  } else {
    *reinterpret_cast<uint2*>(p) = c;
  }
}

// Four bytes packed little-endian into one word.
__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  return c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
}

// clamp(RNE(v), -127, 127) as a byte.
__device__ __forceinline__ uint32_t int8_code(float v) {
  const float r = __builtin_amdgcn_fmed3f(__builtin_rintf(v), -127.0f, 127.0f);
  return (uint32_t)((int32_t)r) & 0xFFu;
}

template <bool kTiny>
__device__ __forceinline__ uint2 int8_chunk(uint4 w, const BlockDiv& d) {
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t out[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint32_t w0 = ws[2 * h], w1 = ws[2 * h + 1];
    out[h] = pack4(int8_code(div_block<kTiny>(bf16_lo(w0), d)),
                   int8_code(div_block<kTiny>(bf16_hi(w0), d)),
                   int8_code(div_block<kTiny>(bf16_lo(w1), d)),
                   int8_code(div_block<kTiny>(bf16_hi(w1), d)));
  }
  return make_uint2(out[0], out[1]);
}

// int8 chunk for any row: an all-zero row (s == 0) has codes 0.
__device__ __forceinline__ uint2 int8_chunk_any(uint4 w, float s, const BlockDiv& d) {
  if (s == 0.0f) return make_uint2(0u, 0u);
  return d.tiny ? int8_chunk<true>(w, d) : int8_chunk<false>(w, d);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

}  // namespace prr

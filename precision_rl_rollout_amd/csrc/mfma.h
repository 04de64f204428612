// MFMA, fragment and buffer-load helpers shared by the GEMM kernels
// (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "prr_device.h"

namespace prr {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4f mfma_fp8(const v8i& w, const v8i& a) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // Scale operands 0 select the unscaled encoding of the instruction;
  // format fields 0 / 0 select fp8 e4m3 for both operands.
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(w, a, zero, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ v4i mfma_i8x2(const v8i& w, const v8i& a, v4i acc) {
  const v4i wl = {w[0], w[1], w[2], w[3]}, wh = {w[4], w[5], w[6], w[7]};
  const v4i al = {a[0], a[1], a[2], a[3]}, ah = {a[4], a[5], a[6], a[7]};
  acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(wl, al, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(wh, ah, acc, 0, 0, 0);
}

// Four fp32 results for C[m, n..n+3] -> bf16, bounds-checked store.
__device__ __forceinline__ void store4(uint16_t* C, int64_t M, int64_t N, int64_t m, int64_t n,
                                       const float v[4]) {
  if (m >= M) return;
  uint16_t* p = C + m * N + n;
  if (n + 3 < N && (N & 3) == 0) {
    const uint32_t lo = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
    const uint32_t hi = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = make_uint2(lo, hi);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) p[r] = (uint16_t)f32_to_bf16_rne(v[r]);
  }
}

// Buffer resource (V#) over `bytes` bytes at `base`: raw loads at offsets
// beyond the range return zeros, so tiles that run past M or N need no
// per-lane branch (branches around loads would also force the compiler to
// wait for every outstanding load before the first MFMA).
// Base and size must be the same for the whole wave; they pass through
// readfirstlane so the compiler knows it (a descriptor it cannot prove
// uniform turns every load into a loop over lanes).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const int n = __builtin_amdgcn_readfirstlane((int)(bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes));
  void* p = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, n, 0x00020000);
}

// 32 bytes of one operand row for one 128-deep block: bytes [16 g, 16 g + 16)
// and [64 + 16 g, 64 + 16 g + 16) of the block, g = lane / 16 (so 4
// consecutive lanes read 64 contiguous bytes).  Weight and activation
// fragments are always filled the same way.
// An offset past every buffer range (ranges are below 2^31 bytes).
constexpr int kOutOfRange = 0x7FFFFFFF & ~0xFF;

__device__ __forceinline__ v8i buffer_load32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(r, voff + 64, soff, 0);
  return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// LDS the skinny kernel may use for its staged FP8 activation scales
// (64 rows x K/128 floats: K up to 81,920 at 64 rows).
constexpr int kSkinnyLdsBytes = 160 * 1024;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// Buffer descriptor as four scalar words (raw buffer, no stride, dword data
// format): base, num_records = bytes (clamped to 2^31 - 1).
__device__ __forceinline__ v4i sgpr_rsrc(const void* base, int64_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  v4i r;
  r[0] = (int)__builtin_amdgcn_readfirstlane((uint32_t)b);
  r[1] = (int)(__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) & 0xFFFFu);
  r[2] = __builtin_amdgcn_readfirstlane((int)(bytes > 0x7FFFFFFF ? 0x7FFFFFFF : bytes));
  r[3] = 0x00020000;
  return r;
}

// Direct-to-LDS buffer loads: lane l's 16 (4) bytes land at LDS byte address
// lds + 16 l (4 l); offsets at or past num_records read zeros.  Issued as
// inline assembly so that the compiler adds no wait of its own on them
// before LDS reads (its alias tracking of such loads cannot tell ring slots
// or stages apart, and waited for the next slot's loads before reading the
// current one); the kernels wait for them explicitly with s_waitcnt vmcnt.
__device__ __forceinline__ void dma_b128(v4i rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

// The same for data read exactly once (the decode GEMM's weight stream),
// marked non-temporal ("nt"): the L2 keeps it as streaming data, to be
// replaced first, so the lines the kernel reuses (activations, partial
// output lines that later strips of the same XCD complete) stay resident.
// Measured on the decode GEMM with cold weights: 7-9% faster at 32-64
// rows and 2-7% at one row; the scope bits (sc0, sc1) made no difference.
__device__ __forceinline__ void dma_b128_stream(v4i rsrc, uint32_t lds, int voff, int soff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}

__device__ __forceinline__ void dma_b32(v4i rsrc, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}

// s_waitcnt immediate for vmcnt(n), n < 64, with expcnt and lgkmcnt left at
// their maxima (no wait on them).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier that orders LDS only.  __syncthreads() also fences
// global memory, which waits for every outstanding global load and would
// drain the load pipelines below at each barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace prr

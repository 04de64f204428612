// Decode attention over the FP8 KV cache ("FP8-RL: A Practical and Stable
// Low-Precision Stack for LLM Reinforcement Learning", abstract, item (ii):
// FP8 KV cache with per-step Q/K/V scales).  One new token per sequence;
// query head h reads cache head h / (Hq / Hkv).  The query is quantized with
// its per-tensor scale by the library's e4m3 encoder; score of cached token
// t: s_q s_k c (q^ . k^_t); softmax over the sequence's tokens; output
// s_v sum_t p_t v^_t, rounded once to bf16.
//
// Bound by HBM: every cached token costs 2 x 128 bytes per KV head (its K
// and V codes) against ~5 flops per byte for a group of 5 query heads, so
// the arithmetic runs on the vector ALUs (fp32), not on MFMA.
//
//  * One 512-thread workgroup per (sequence, KV head).  16 lanes take one
//    token (8 of its 128 dimensions each: one 8-byte load of K and one of
//    V), a wave takes 4 tokens per step and 8 steps (32 tokens) per
//    iteration, with all 16 loads of an iteration issued before any math.
//    Wave w takes iterations w, w + 8, ... of the sequence.
//  * The decoded query of every head of the group stays in registers
//    (8 G floats per lane).  Dot products are reduced over the 16 lanes of
//    a token by butterflies.
//  * Online softmax in the base-2 domain (scores carry log2 e), updated once
//    per iteration: a wave keeps the running maximum and sum per head and a
//    partial output per lane (its own tokens), rescaled when the maximum
//    grows; the 8 waves are combined through LDS at the end.
//  * The sequence's block-table row is staged in LDS (2048 pages at a time).
//    A token whose page entry is negative or points past the cache is
//    skipped; the loads of skipped and padding tokens are not issued.
#include "launch.h"
#include "prr_device.h"

namespace prr {

constexpr int kAttThreads = 512;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kAttD = 128;            // head dimension
constexpr int kAttSteps = 8;          // 4-token steps per iteration
constexpr int kAttIter = 4 * kAttSteps;
constexpr int kAttTablePages = 2048;  // block-table entries staged at a time
constexpr float kLog2e = 1.4426950408889634f;

// Eight e4m3 codes -> eight floats (exact).
__device__ __forceinline__ void decode8(uint2 c, float f[8]) {
  const uint32_t w[2] = {c.x, c.y};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], true);
    f[4 * h + 0] = lo[0];
    f[4 * h + 1] = lo[1];
    f[4 * h + 2] = hi[0];
    f[4 * h + 3] = hi[1];
  }
}

// Sum over the 16 lanes of a row, left in every lane of the row: DPP
// exchanges within quads, then half-rows, then rows (ALU only; a shuffle
// through LDS costs a round trip per step).
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Values that are uniform within each 16-lane row: combine the 4 rows
// through scalar reads of lanes 0, 16, 32, 48.
__device__ __forceinline__ float rows_max4(float v) {
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float rows_sum4(float v) {
  float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);   // row_half_mirror
  v += dpp_mov<0x140>(v);   // row_mirror
  return v;
}

template <int G>
__global__ __launch_bounds__(kAttThreads) void fp8_decode_attention_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k_cache, const uint8_t* __restrict__ v_cache,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hq,
    int Hkv, int page, int max_blocks, int64_t num_slots, float softmax_scale,
    uint16_t* __restrict__ out) {
  __shared__ int32_t tbl[kAttTablePages];
  __shared__ float part[kAttWaves][G][kAttD + 2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int b = blockIdx.x / Hkv, kvh = blockIdx.x - b * Hkv;
  const int tg = lane >> 4, l16 = lane & 15;       // token in the step, dims 8 l16 ..
  const int64_t row_bytes = (int64_t)Hkv * kAttD;
  uint16_t* ob = out + ((int64_t)b * Hq + (int64_t)kvh * G) * kAttD;

  int64_t n = seq_lens[b];
  n = n < 0 ? 0 : n;
  n = min(n, (int64_t)max_blocks * page);
  if (n == 0) {
    for (int e = tid; e < G * kAttD; e += kAttThreads) ob[e] = 0;
    return;
  }

  // The group's query heads: quantized with s_q, decoded (exact).
  const float sq = *q_scale;
  const BlockDiv dq = block_div(sq);
  float qv[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint16_t* qh = q + ((int64_t)b * Hq + (int64_t)kvh * G + g) * kAttD + 8 * l16;
    const uint4 w = *reinterpret_cast<const uint4*>(qh);
    decode8(e4m3_chunk_any<true>(w, sq, dq), qv[g]);
  }
  // Score scale in the base-2 domain.
  const float cs = sq * (*k_scale) * softmax_scale * kLog2e;
  const float sv = *v_scale;

  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = -__builtin_inff();
    l[g] = 0.f;
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[g][d] = 0.f;
  }

  const int32_t* trow = block_table + (int64_t)b * max_blocks;
  const int64_t chunk_tokens = (int64_t)kAttTablePages * page;
  for (int64_t c0 = 0; c0 < n; c0 += chunk_tokens) {
    const int64_t c1 = min(n, c0 + chunk_tokens);
    const int p0 = (int)(c0 / page);
    const int np = (int)((c1 - c0 + page - 1) / page);
    __syncthreads();                                   // previous chunk's readers are done
    for (int e = tid; e < np; e += kAttThreads) tbl[e] = trow[p0 + e];
    __syncthreads();
    const int64_t iters = (c1 - c0 + kAttIter - 1) / kAttIter;
    for (int64_t it = wave; it < iters; it += kAttWaves) {
      const int64_t t0 = c0 + it * kAttIter;
      uint2 kc[kAttSteps], vc[kAttSteps];
      bool ok[kAttSteps];
#pragma unroll
      for (int u = 0; u < kAttSteps; ++u) {
        const int64_t t = t0 + 4 * u + tg;
        int64_t slot = -1;
        if (t < c1) {
          // 32-bit offset within the staged chunk (c0 is a whole number of
          // pages): a 64-bit division here costs ~100 instructions a token
          const uint32_t rel = (uint32_t)(t - c0);
          const uint32_t pi = rel / (uint32_t)page;
          const int pg = tbl[pi];
          slot = (int64_t)pg * page + (rel - pi * (uint32_t)page);
        }
        ok[u] = slot >= 0 && slot < num_slots;
        kc[u] = make_uint2(0, 0);
        vc[u] = make_uint2(0, 0);
        if (ok[u]) {
          const int64_t off = slot * row_bytes + (int64_t)kvh * kAttD + 8 * l16;
          kc[u] = *reinterpret_cast<const uint2*>(k_cache + off);
          vc[u] = *reinterpret_cast<const uint2*>(v_cache + off);
        }
      }
      // Scores (base 2) of this lane's tokens, for every head.
      float s[kAttSteps][G];
#pragma unroll
      for (int u = 0; u < kAttSteps; ++u) {
        float kf[8];
        decode8(kc[u], kf);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float dot = 0.f;
#pragma unroll
          for (int d = 0; d < 8; ++d) dot = __builtin_fmaf(qv[g][d], kf[d], dot);
          dot = row_sum16(dot);
          s[u][g] = ok[u] ? dot * cs : -__builtin_inff();
        }
      }
      // Softmax update per head (s becomes p in place), then one decode of
      // each token's V for all heads.
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float mi = s[0][g];
#pragma unroll
        for (int u = 1; u < kAttSteps; ++u) mi = fmaxf(mi, s[u][g]);
        mi = rows_max4(mi);
        const float mn = fmaxf(m[g], mi);
        // (every token so far skipped: mn = -inf; subtract 0 so that the
        // weights and alpha come out 0 rather than NaN)
        const float mref = mn == -__builtin_inff() ? 0.f : mn;
        const float alpha = __builtin_amdgcn_exp2f(m[g] - mref);
        m[g] = mn;
        float ps = 0.f;
#pragma unroll
        for (int u = 0; u < kAttSteps; ++u) {
          s[u][g] = __builtin_amdgcn_exp2f(s[u][g] - mref);
          ps += s[u][g];
        }
        ps = rows_sum4(ps);
        l[g] = l[g] * alpha + ps;
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[g][d] *= alpha;
      }
#pragma unroll
      for (int u = 0; u < kAttSteps; ++u) {
        float vf[8];
        decode8(vc[u], vf);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
          for (int d = 0; d < 8; ++d) acc[g][d] = __builtin_fmaf(s[u][g], vf[d], acc[g][d]);
      }
    }
  }

  // The 4 token groups of a wave, then the 8 waves.
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      acc[g][d] += __shfl_xor(acc[g][d], 16, 64);
      acc[g][d] += __shfl_xor(acc[g][d], 32, 64);
    }
  if (lane < 16) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int d = 0; d < 8; ++d) part[wave][g][8 * lane + d] = acc[g][d];
      if (lane == 0) {
        part[wave][g][kAttD] = m[g];
        part[wave][g][kAttD + 1] = l[g];
      }
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kAttD; e += kAttThreads) {
    const int g = e / kAttD, d = e - g * kAttD;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, part[w][g][kAttD]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kAttWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(part[w][g][kAttD] - M);
        L += part[w][g][kAttD + 1] * f;
        O += part[w][g][d] * f;
      }
    }
    const float v = L > 0.f ? sv * (O / L) : 0.f;
    ob[e] = (uint16_t)f32_to_bf16_rne(v);
  }
}

hipError_t launch_fp8_decode_attention(const uint16_t* q, const float* q_scale,
                                       const uint8_t* k_cache, const uint8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       int64_t B, int64_t Hq, int64_t Hkv, int64_t page,
                                       int64_t max_blocks, int64_t num_slots,
                                       float softmax_scale, uint16_t* out, hipStream_t stream) {
  const int G = (int)(Hq / Hkv);
  const dim3 grid((unsigned)(B * Hkv));
#define PRR_ATT(GV)                                                                          \
  case GV:                                                                                   \
    hipLaunchKernelGGL((fp8_decode_attention_kernel<GV>), grid, dim3(kAttThreads), 0, stream, \
                       q, q_scale, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, \
                       (int)Hq, (int)Hkv, (int)page, (int)max_blocks, num_slots,             \
                       softmax_scale, out);                                                  \
    break;
  switch (G) {
    PRR_ATT(1)
    PRR_ATT(2)
    PRR_ATT(3)
    PRR_ATT(4)
    PRR_ATT(5)
    PRR_ATT(6)
    PRR_ATT(7)
    PRR_ATT(8)
    default:
      return hipErrorInvalidValue;
  }
#undef PRR_ATT
  return hipGetLastError();
}

}  // namespace prr

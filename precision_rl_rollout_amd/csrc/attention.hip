// Decode attention over the FP8 KV cache ("FP8-RL: A Practical and Stable
// Low-Precision Stack for LLM Reinforcement Learning", abstract, item (ii):
// FP8 KV cache with per-step Q/K/V scales).  One new token per sequence;
// query head h reads cache head h / (Hq / Hkv).  The query is quantized with
// its per-tensor scale by the library's e4m3 encoder; score of cached token
// t: s_q s_k c (q^ . k^_t); softmax over the sequence's tokens; output
// s_v sum_t p_t v^_t, rounded once to bf16.
//
// Bound by HBM: every cached token costs 2 x 128 bytes per KV head (its K
// and V codes) against ~5 flops per byte for a group of 5 query heads.
//
//  * One 512-thread workgroup per (sequence, KV head); wave w takes
//    iterations w, w + 8, ... of the sequence, 32 tokens (two tiles of 16)
//    an iteration, with every load of an iteration issued before any math.
//  * Q K^T on the matrix cores in bf16: e4m3 -> bf16 is exact, and the bf16
//    16x16x32 instruction sums its products to fp32 accuracy, while the
//    e4m3 instructions of gfx950 keep only ~13 bits inside a dot product
//    (measured: errors up to 2e-4 of the sum of |products|), which the
//    softmax would turn into output errors well above a bf16 rounding.  One
//    tile of 16 tokens against the group's query heads (rows past G zero) is
//    four instructions, with no cross-lane reduction.
//  * Online softmax in the base-2 domain (scores carry log2 e), updated once
//    per iteration per head; P V on the vector ALUs in fp32 with the
//    probabilities passed through a per-wave LDS tile; the 8 waves are
//    combined through LDS at the end.
//  * The sequence's block-table row is staged in LDS (2048 pages at a time).
//    A token whose page entry is negative or points past the cache is
//    skipped; the loads of skipped and padding tokens are not issued.
#include "launch.h"
#include "prr_device.h"

namespace prr {

constexpr int kAttThreads = 512;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kAttD = 128;            // head dimension
constexpr int kAttIter = 32;          // tokens of a wave iteration (two tiles of 16)
constexpr int kAttTablePages = 2048;  // block-table entries staged at a time
constexpr int kAttOrderMax = 256;     // sequences ordered by length in-kernel (at most)
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

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Eight e4m3 codes -> eight bf16 values (exact: every e4m3 value, subnormals
// included, is a bf16 value), in code order.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const uint4 r = make_uint4(
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)));
  return __builtin_bit_cast(v8bf, r);
}

// x / d for x < 2^24 and a quotient below 2^6 (x at most 32 past a
// multiple of d): one float product, corrected by one step either way.
__device__ __forceinline__ uint32_t small_div(uint32_t x, uint32_t d, float inv_d) {
  uint32_t qt = (uint32_t)((float)x * inv_d);
  const int32_t rem = (int32_t)(x - qt * d);
  if (rem < 0) --qt;
  else if (rem >= (int32_t)d) ++qt;
  return qt;
}

template <int G>
__global__ __launch_bounds__(kAttThreads) void fp8_decode_attention_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k_cache, const uint8_t* __restrict__ v_cache,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hq,
    int Hkv, int page, int max_blocks, int64_t num_slots, float softmax_scale,
    uint16_t* __restrict__ out) {
  constexpr int kPS = G <= 4 ? 4 : 8;               // pbuf row stride (heads)
  __shared__ int64_t tbase[kAttTablePages];        // byte offset of a staged page's first row
  __shared__ int32_t tlim[kAttTablePages];         // its slots inside the cache (0: skipped)
  __shared__ float part[kAttWaves][G][kAttD + 2];
  __shared__ float4 pbuf[kAttWaves][kAttIter][kPS / 4];  // [token of the iteration][head]
  __shared__ int32_t pick;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = (int)(gridDim.x / Hkv);
  const int kvh = blockIdx.x % Hkv;
  const int64_t n_cap = (int64_t)max_blocks * page;
  auto length = [&](int bb) -> int64_t {
    const int64_t v = seq_lens[bb];
    return min(v < 0 ? (int64_t)0 : v, n_cap);
  };
  // Longest sequences first: workgroup i serves the sequence of rank i / Hkv
  // in order of decreasing length (ties by index), so that the work left
  // for the last workgroups to start is the shortest.  The ranks are a
  // permutation, so exactly one thread finds the target.
  int b = (int)(blockIdx.x / Hkv);
  if (B <= kAttOrderMax) {
    const int64_t* lens = tbase;                   // staging space until the table is loaded
    for (int e = tid; e < B; e += kAttThreads) tbase[e] = length(e);
    __syncthreads();
    for (int j = tid; j < B; j += kAttThreads) {
      const int64_t lj = lens[j];
      int rank = 0;
      for (int i = 0; i < B; ++i) rank += (lens[i] > lj) || (lens[i] == lj && i < j);
      if (rank == b) pick = j;
    }
    __syncthreads();
    b = pick;
  }
  // MFMA layout: lane (g, r) = row r (token r of a 16-token tile, or query
  // head r), dimensions [32 g, 32 g + 32) as 4 slices of 8 (one per
  // 16x16x32 instruction); its results are tokens 4 g .. 4 g + 3 of head r.
  // V layout: lane (tg, dg) = tokens 4 tg .. 4 tg + 3 of a tile, dimensions
  // [8 dg, 8 dg + 8).
  const int g = lane >> 4, r = lane & 15;
  const int tg = g, dg = r;
  const uint32_t row_bytes = (uint32_t)Hkv * kAttD;
  const uint8_t* kbase = k_cache + (int64_t)kvh * kAttD;
  const uint8_t* vbase = v_cache + (int64_t)kvh * kAttD + 8 * dg;
  uint16_t* ob = out + ((int64_t)b * Hq + (int64_t)kvh * G) * kAttD;

  // (no cache slots: every token is skipped)
  const int64_t n = num_slots > 0 ? length(b) : 0;
  if (n == 0) {
    for (int e = tid; e < G * kAttD; e += kAttThreads) ob[e] = 0;
    return;
  }

  // The group's query heads, quantized with s_q and decoded to bf16 (exact):
  // second MFMA operand, row r = head r (zero past the group).  Slice j of
  // lane (g, r) holds dimensions [32 g + 8 j, 32 g + 8 j + 8).
  const float sq = *q_scale;
  const BlockDiv dq = block_div(sq);
  v8bf qf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) qf[j] = __builtin_bit_cast(v8bf, make_uint4(0, 0, 0, 0));
  if (r < G) {
    const uint16_t* qh = q + ((int64_t)b * Hq + (int64_t)kvh * G + r) * kAttD + 32 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint2 c = e4m3_chunk_any<true>(*reinterpret_cast<const uint4*>(qh + 8 * j), sq, dq);
      qf[j] = e4m3x8_to_bf16(c.x, c.y);
    }
  }
  // Score scale in the base-2 domain.
  const float cs = sq * (*k_scale) * softmax_scale * kLog2e;
  const float sv = *v_scale;
  const float inv_page = 1.0f / (float)page;

  float m = -__builtin_inff(), l = 0.f;              // head r (equal in the 4 lanes of r)
  float acc[G][8];                                  // this lane's tokens and dimensions
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[h][d] = 0.f;

  const int32_t* trow = block_table + (int64_t)b * max_blocks;
  const int64_t chunk_tokens = (int64_t)kAttTablePages * page;
  for (int64_t c0 = 0; c0 < n; c0 += chunk_tokens) {
    const int64_t c1 = min(n, c0 + chunk_tokens);
    const int p0 = (int)(c0 / page);
    const int np = (int)((c1 - c0 + page - 1) / page);
    __syncthreads();                                   // previous readers of the table are done
    for (int e = tid; e < np; e += kAttThreads) {
      const int64_t pid = trow[p0 + e];
      const int64_t first = pid * page;
      const int64_t lim = pid < 0 ? 0 : min((int64_t)page, max((int64_t)0, num_slots - first));
      tlim[e] = (int32_t)lim;
      tbase[e] = lim > 0 ? first * row_bytes : 0;
    }
    __syncthreads();
    const int iters = (int)((c1 - c0 + kAttIter - 1) / kAttIter);
    const int ntok = (int)(c1 - c0);
    for (int it = wave; it < iters; it += kAttWaves) {
      // Token k of the iteration is token 32 it + k of the chunk: page
      // pi0 + (off0 + k) / page of the staged table, all in 32 bits (a
      // chunk holds at most 2^31 tokens).  A token that is absent (past the
      // length, or its slot outside the cache) reads row 0 of the cache
      // (there is one) and is masked.
      const uint32_t rel0 = (uint32_t)it * kAttIter;
      const uint32_t pi0 = rel0 / (uint32_t)page, off0 = rel0 - pi0 * (uint32_t)page;
      auto locate = [&](int k, uint64_t& at) -> bool {
        const bool in = (int)rel0 + k < ntok;
        const uint32_t off = off0 + (uint32_t)k;
        const uint32_t qp = small_div(off, (uint32_t)page, inv_page);
        const uint32_t pi = in ? pi0 + qp : 0;
        const uint32_t o = off - qp * (uint32_t)page;
        // (pi is in range either way; the empty asm keeps the compiler from
        // moving the reads under a branch on ok)
        int32_t lim = tlim[pi];
        int64_t base = tbase[pi];
        asm volatile("" : "+v"(lim), "+v"(base));
        const bool ok = in & ((int32_t)o < lim);
        at = ok ? (uint64_t)base + (uint64_t)o * row_bytes : 0;
        return ok;
      };
      uint4 kl[2], kh[2];                               // bytes [32 g, 32 g + 32) of token r
      uint2 vc[2][4];
      uint64_t okm[2];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        uint64_t at;
        const bool ok = locate(16 * tile + r, at);
        okm[tile] = __ballot(ok) & 0xFFFF;               // bit j: token 16 tile + j
        const uint8_t* kp = kbase + at + 32 * g;
        kl[tile] = *reinterpret_cast<const uint4*>(kp);
        kh[tile] = *reinterpret_cast<const uint4*>(kp + 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool okv = locate(16 * tile + 4 * tg + i, at);
          const uint2 v = *reinterpret_cast<const uint2*>(vbase + at);
          vc[tile][i] = make_uint2(okv ? v.x : 0u, okv ? v.y : 0u);
        }
      }
      // Scores (base 2): lane (g, r) gets tokens 16 tile + 4 g + i of head r.
      float sc[2][4];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        v4f d = {0.f, 0.f, 0.f, 0.f};
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kl[tile].x, kl[tile].y), qf[0], d,
                                                    0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kl[tile].z, kl[tile].w), qf[1], d,
                                                    0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kh[tile].x, kh[tile].y), qf[2], d,
                                                    0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kh[tile].z, kh[tile].w), qf[3], d,
                                                    0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[tile][i] = ((okm[tile] >> (4 * g + i)) & 1) ? d[i] * cs : -__builtin_inff();
      }
      float mi = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      mi = fmaxf(mi, __shfl_xor(mi, 16, 64));
      mi = fmaxf(mi, __shfl_xor(mi, 32, 64));
      const float mn = fmaxf(m, mi);
      // (every token so far skipped: mn = -inf; subtract 0 so that the
      // weights and alpha come out 0 rather than NaN)
      const float mref = mn == -__builtin_inff() ? 0.f : mn;
      const float alpha = __builtin_amdgcn_exp2f(m - mref);
      m = mn;
      float ps = 0.f;
      float* prow = reinterpret_cast<float*>(&pbuf[wave][0][0]);
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = __builtin_amdgcn_exp2f(sc[tile][i] - mref);
          ps += pv;
          if (r < G) prow[(16 * tile + 4 * g + i) * kPS + r] = pv;
        }
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      l = l * alpha + ps;
      // Rescale, then P V in the V layout.  The probabilities were written
      // by this wave; its LDS operations complete in order.
      asm volatile("" ::: "memory");
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ah = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, alpha), h));
#pragma unroll
        for (int d = 0; d < 8; ++d) acc[h][d] *= ah;
      }
#pragma unroll
      for (int tile = 0; tile < 2; ++tile)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = 16 * tile + 4 * tg + i;
          float pt[kPS];
#pragma unroll
          for (int c = 0; c < kPS / 4; ++c) {
            const float4 p4 = pbuf[wave][k][c];
            pt[4 * c + 0] = p4.x;
            pt[4 * c + 1] = p4.y;
            pt[4 * c + 2] = p4.z;
            pt[4 * c + 3] = p4.w;
          }
          float vf[8];
          decode8(vc[tile][i], vf);
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int d = 0; d < 8; ++d) acc[h][d] = __builtin_fmaf(pt[h], vf[d], acc[h][d]);
        }
      asm volatile("" ::: "memory");
    }
  }

  // The 4 token groups of a wave, then the 8 waves.
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      acc[h][d] += __shfl_xor(acc[h][d], 16, 64);
      acc[h][d] += __shfl_xor(acc[h][d], 32, 64);
    }
  if (tg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int d = 0; d < 8; ++d) part[wave][h][8 * dg + d] = acc[h][d];
    if (r < G) {
      part[wave][r][kAttD] = m;
      part[wave][r][kAttD + 1] = l;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kAttD; e += kAttThreads) {
    const int h = e / kAttD, d = e - h * kAttD;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, part[w][h][kAttD]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kAttWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(part[w][h][kAttD] - M);
        L += part[w][h][kAttD + 1] * f;
        O += part[w][h][d] * f;
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

// W8A8 linear layers on gfx950 MFMA, bf16 output.
//
// FP8 (FP8-RL, abstract, item (i): blockwise FP8 W8A8 linear layers):
//   C[m, n] = sum_kb sa[m, kb] * sw[n/128, kb] * P(m, n, kb),
//   P = sum over the 128 k of block kb of D(Aq[m, k]) D(Wq[n, k]).
// One v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-deep scale block,
// so P comes out of a single MFMA with a zero accumulator and is folded
// into the fp32 accumulator with one FMA by sa * sw.
//
// INT8 (FlashRL article, INT8 rollout): v_mfma_i32_16x16x64_i8 accumulates
// the exact int32 dot product over all of K; the per-row and per-channel
// scales are applied once, in the epilogue.
//
// Operand roles.  The weight fragment is the MFMA's first operand and the
// activation fragment its second, so each lane's four accumulators hold
// four consecutive output channels n of one token m: one activation scale
// per lane per block, and 8-byte bf16 stores.
//
// Fragment layout.  For both MFMAs a lane holds, for operand row (l mod 16),
// bytes [16 g, 16 g + 16) and [64 + 16 g, 64 + 16 g + 16) of the 128-byte
// block, g = l / 16 (so 4 consecutive lanes read 64 contiguous bytes).  The
// two operands are filled the same way, so whatever order the instruction
// walks its k in, every product pairs A[m, k] with W[n, k] for the same k
// and each k of the block is used once.
#include <algorithm>

#include "launch.h"
#include "mfma.h"
#include "prr_device.h"

namespace prr {

// ---------------------------------------------------------------------------
// Skinny-M path (M <= 64 where the persistent decode kernel cannot hold the
// activations in registers, i.e. long K).  The weight is streamed from HBM once and
// is the whole cost: every design choice below serves keeping enough weight
// bytes in flight per CU.
//
// A workgroup is 4 waves arranged as (4 / KS) channel groups x KS K-groups.
// A wave owns S strips of 16 output channels and all MT m-tiles of 16
// tokens; K-group g takes K blocks g, g + KS, g + 2 KS, ...  Per K block a
// wave loads its S weight fragments and MT activation fragments (32 bytes
// per lane each) into a D-deep register ring, so D blocks of loads are in
// flight while the MFMAs of the oldest block run.  The KS partial sums of a
// channel group are added through LDS at the end.  Activations (at most
// 64 x K bytes) stay in L2 and are re-read by every strip; the weight is
// read exactly once.
// ---------------------------------------------------------------------------
template <int MT, int S, int KS, int D>
struct SkinnyCfg {
  static constexpr int kMT = MT, kS = S, kKS = KS, kD = D;
  static constexpr int kGroups = 4 / KS;                 // channel groups per workgroup
  static constexpr int kCols = kGroups * S * 16;         // output channels per workgroup
  static_assert(KS == 1 || KS == 2 || KS == 4, "KS divides 4");
  static_assert(S * 16 <= 128 && (128 % (S * 16)) == 0, "a wave's strips lie in one 128-block");
  static_assert(KS == 1 || S * MT <= 16, "the reduction buffer stays within 64 KB of LDS");
};

// Configuration per m-tile count, chosen by a sweep of (S, KS, D) on MI355X
// over N = 27648 / 37888, K = 5120 / 3584, M = 1 .. 64 (FP8 and INT8).
template <int MT> struct SkinnyPick;
template <> struct SkinnyPick<1> { using type = SkinnyCfg<1, 2, 4, 2>; };
template <> struct SkinnyPick<2> { using type = SkinnyCfg<2, 4, 4, 2>; };
template <> struct SkinnyPick<3> { using type = SkinnyCfg<3, 4, 4, 2>; };
template <> struct SkinnyPick<4> { using type = SkinnyCfg<4, 4, 2, 2>; };

// Narrow layers (few output channels, long K: e.g. a down projection, N 5120
// x K 27648): the configurations above give a workgroup 32-128 channels,
// which leaves most CUs idle when N is small (40 workgroups for 5120
// channels at MT 4).  Here a workgroup takes one 16-channel strip with K
// split over its 4 waves and a 4-deep ring, so there is one workgroup per
// strip; each re-reads the activations (M x K from L2) once.
template <int MT> struct SkinnyNarrow { using type = SkinnyCfg<MT, 1, 4, 4>; };

template <class Cfg, bool kInt8>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ C) {
  constexpr int MT = Cfg::kMT, S = Cfg::kS, KS = Cfg::kKS, D = Cfg::kD;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kg = wave % KS, cg = wave / KS;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * Cfg::kCols + cg * (S * 16);   // wave's first channel
  const int KB = (int)(K / kBlock);
  const int nk = (KB - kg + KS - 1) / KS;                                // K blocks of this wave
  // A wave whose strips all lie past N (possible in the last workgroup)
  // reads nothing (empty resource); it still joins the reduction.
  const bool wave_live = n0 < N;                                         // wave-uniform
  const int64_t wrows = wave_live ? min<int64_t>(S * 16, N - n0) : 0;
  const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + (wave_live ? n0 : 0) * K, wrows * K);
  const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(A, M * K);
  // (a dead wave reads the scales of channel block 0: finite values that
  // multiply its all-zero products)
  const float* swp = sw + (wave_live ? (n0 >> 7) * KB : 0) + kg;

  // Dynamic LDS, used twice: first for the FP8 activation scales of all
  // MT * 16 token rows, transposed to [K block][row] so that the 16 rows of
  // a fragment are 16 consecutive words; then, after a barrier, for the
  // cross-wave reduction of the K-split partial sums.
  extern __shared__ float lds_dyn[];
  float* lsa = lds_dyn;
  if constexpr (!kInt8) {
    const int rows = MT * 16;
    for (int e = threadIdx.x; e < rows * KB; e += 256) {
      const int m = e / KB, kb = e - m * KB;
      lsa[kb * rows + m] = (m < M) ? sa[(int64_t)m * KB + kb] : 0.f;
    }
    __syncthreads();
  }

  int woff[S], aoff[MT];
#pragma unroll
  for (int s = 0; s < S; ++s) woff[s] = (int)((s * 16 + r16) * K) + g * 16 + kg * kBlock;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) aoff[mt] = (int)((mt * 16 + r16) * K) + g * 16 + kg * kBlock;

  float accf[S][MT][4];
  v4i acci[S][MT];
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acci[s][mt] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[s][mt][r] = 0.f;
    }

  // D-deep register ring of weight and activation fragments.  The stream
  // holds nothing but these 16-byte loads and is issued in stage order, so
  // the wait before a stage's MFMAs lets the younger D - 1 stages stay in
  // flight.  Stages past the wave's last K block are loaded at an offset
  // outside every buffer (no memory traffic, zeros returned) and their
  // MFMAs add zeros, which keeps the pipeline free of branches.
  v8i wbuf[D][S], abuf[D][MT];
  auto load_stage = [&](int d, int i) {
    const int kofs = (i < nk) ? i * (KS * kBlock) : kOutOfRange;     // wave-uniform
#pragma unroll
    for (int s = 0; s < S; ++s) wbuf[d][s] = buffer_load32(wres, woff[s] + kofs, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) abuf[d][mt] = buffer_load32(ares, aoff[mt] + kofs, 0);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_stage(d, d);
    __builtin_amdgcn_sched_barrier(0);
  }

  for (int t = 0; t < nk; t += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = t + d;
      if constexpr (kInt8) {
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acci[s][mt] = mfma_i8x2(wbuf[d][s], abuf[d][mt], acci[s][mt]);
      } else {
        const int ic = min(i, nk - 1);
        const float swv = swp[ic * KS];
        const float* srow = lsa + (kg + ic * KS) * (MT * 16) + r16;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const v4f p = mfma_fp8(wbuf[d][s], abuf[d][mt]);
            const float sc = srow[mt * 16] * swv;
#pragma unroll
            for (int r = 0; r < 4; ++r) accf[s][mt][r] = fmaf(p[r], sc, accf[s][mt][r]);
          }
      }
      load_stage(d, i + D);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // Add the KS partial sums of each channel group (int32 partials are
  // stored bit-cast in the same array) and store.
  if constexpr (KS > 1) {
    if constexpr (!kInt8) __syncthreads();          // every wave is done with lsa
    auto red = reinterpret_cast<float (*)[S][MT][4][64]>(lds_dyn);
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[wave][s][mt][r][lane] = kInt8 ? __int_as_float(acci[s][mt][r]) : accf[s][mt][r];
    __syncthreads();
    if (kg != 0) return;
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
          for (int j = 1; j < KS; ++j) {
            if constexpr (kInt8)
              acci[s][mt][r] += __float_as_int(red[wave + j][s][mt][r][lane]);
            else
              accf[s][mt][r] += red[wave + j][s][mt][r][lane];
          }
  }
  // INT8: the row and channel scales this lane applies, loaded together
  // and branch-free (clamped indices, zero past M or N), so the stores
  // below wait for one round trip rather than one per fragment.
  float smv[MT], snv[S][4];
  if constexpr (kInt8) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = mt * 16 + r16;
      const float x = sa[min(m, (int64_t)M - 1)];
      smv[mt] = m < M ? x : 0.f;
    }
#pragma unroll
    for (int s = 0; s < S; ++s)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = (int64_t)n0 + s * 16 + 4 * g + r;
        const float x = sw[min(n, (int64_t)N - 1)];
        snv[s][r] = n < N ? x : 0.f;
      }
  }
#pragma unroll
  for (int s = 0; s < S; ++s)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int64_t m = mt * 16 + r16;
      const int64_t n = n0 + s * 16 + 4 * g;
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (kInt8) {
          v[r] = (float)acci[s][mt][r] * (smv[mt] * snv[s][r]);
        } else {
          v[r] = accf[s][mt][r];
        }
      }
      store4(C, M, N, m, n, v);
    }
}

__global__ void fill_zero_bf16_kernel(uint16_t* __restrict__ C, int64_t count) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) C[i] = 0;
}

template <bool kInt8>
static hipError_t launch_gemm(const uint8_t* A, const float* sa, const uint8_t* W,
                              const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* C,
                              hipStream_t stream) {
  if (K == 0) {
    const int64_t count = M * N;
    hipLaunchKernelGGL(fill_zero_bf16_kernel, dim3((unsigned)((count + 255) / 256)), dim3(256), 0,
                       stream, C, count);
    return hipGetLastError();
  }
  {
    hipError_t err = hipSuccess;
    if (launch_gemm_decode<kInt8>(A, sa, W, sw, M, N, K, C, stream, &err)) return err;
  }
  // The skinny kernel addresses A and one 128-row weight slab with 32-bit
  // buffer offsets; its FP8 activation scales (MT x 16 rows x K/128) are
  // staged in LDS.  Above 64 rows the many-token kernel (128-wide tiles when
  // few) is faster.
  const int64_t mt16 = (M + 15) / 16 * 16;
  const size_t skinny_scales = kInt8 ? 0 : (size_t)mt16 * (K / kBlock) * sizeof(float);
  if (M <= 64 && 128 * K < kOutOfRange && M * K < kOutOfRange &&
      skinny_scales <= (size_t)kSkinnyLdsBytes) {
    const int mt = (int)((M + 15) / 16);
    const int cus = compute_units();
#define PRR_SKINNY_LAUNCH(CFG, X)                                                              {                                                                                              using Cfg = CFG;                                                                             const unsigned grid = (unsigned)((N + Cfg::kCols - 1) / Cfg::kCols);                        const size_t lds_red =                                                                           Cfg::kKS > 1 ? (size_t)4 * Cfg::kS * X * 4 * 64 * sizeof(float) : 0;                   const size_t lds = skinny_scales > lds_red ? skinny_scales : lds_red;                       hipLaunchKernelGGL((gemm_skinny_kernel<Cfg, kInt8>), dim3(grid), dim3(256), lds, stream,                        A, sa, W, sw, M, N, K, C);                                              }
#define PRR_SKINNY(X)                                                                          case X:                                                                                        if ((N + SkinnyPick<X>::type::kCols - 1) / SkinnyPick<X>::type::kCols < cus)                   PRR_SKINNY_LAUNCH(typename SkinnyNarrow<X>::type, X)                                       else                                                                                           PRR_SKINNY_LAUNCH(typename SkinnyPick<X>::type, X)                                         break;
    switch (mt) {
      PRR_SKINNY(1)
      PRR_SKINNY(2)
      PRR_SKINNY(3)
      PRR_SKINNY(4)
      default:
        return hipErrorInvalidValue;
    }
#undef PRR_SKINNY
#undef PRR_SKINNY_LAUNCH
    return hipGetLastError();
  }
  {
    hipError_t err = hipSuccess;
    if (launch_gemm_prefill<kInt8>(A, sa, W, sw, M, N, K, C, stream, &err)) return err;
  }
  // Unreachable for shapes the C ABI accepts (K <= kMaxGemmK, grid within
  // range): the many-token kernel takes every such shape the kernels above
  // decline.  Nothing is launched.
  return hipErrorInvalidValue;
}

hipError_t launch_w8a8_block_gemm(const uint8_t* A, const float* sa, const uint8_t* W,
                                  const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* C,
                                  hipStream_t stream) {
  return launch_gemm<false>(A, sa, W, sw, M, N, K, C, stream);
}

hipError_t launch_w8a8_int8_channel_gemm(const int8_t* A, const float* sa, const int8_t* W,
                                         const float* sw, int64_t M, int64_t N, int64_t K,
                                         uint16_t* C, hipStream_t stream) {
  return launch_gemm<true>(reinterpret_cast<const uint8_t*>(A), sa,
                           reinterpret_cast<const uint8_t*>(W), sw, M, N, K, C, stream);
}

}  // namespace prr

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
// the 32 consecutive bytes starting at byte 32 * (l / 16) of the 128-byte
// block.  The two operands are filled the same way, so whatever order the
// instruction walks its k in, every product pairs A[m, k] with W[n, k] for
// the same k and each k of the block is used once.
#include "launch.h"
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

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  v8i r = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  return r;
}

__device__ __forceinline__ v8i zero8() {
  v8i r = {0, 0, 0, 0, 0, 0, 0, 0};
  return r;
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

// ---------------------------------------------------------------------------
// Skinny-M path (decode: M <= 128).  The weight is streamed from HBM once.
// A workgroup of 4 waves owns one 16-channel strip of the output; the waves
// split K into 4 contiguous ranges, each wave runs MT m-tiles of 16 tokens
// over its range, and the 4 partial sums are added through LDS at the end.
// ---------------------------------------------------------------------------
template <int MT, bool kInt8>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ C) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * 16;
  const int64_t KB = K / kBlock;
  const int64_t kb0 = (KB * wave) / 4, kb1 = (KB * (wave + 1)) / 4;

  const int64_t wrow = n0 + r16;
  const bool wvalid = wrow < N;
  const uint8_t* wp = W + wrow * K + g * 32;
  const uint8_t* ap[MT];
  bool avalid[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t m = mt * 16 + r16;
    avalid[mt] = m < M;
    ap[mt] = A + m * K + g * 32;
  }

  float accf[MT][4];
  v4i acci[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) accf[mt][r] = 0.f;
    acci[mt] = v4i{0, 0, 0, 0};
  }

  v8i wf = (wvalid && kb0 < kb1) ? load32(wp + kb0 * kBlock) : zero8();
  for (int64_t kb = kb0; kb < kb1; ++kb) {
    const v8i wcur = wf;
    if (kb + 1 < kb1) wf = wvalid ? load32(wp + (kb + 1) * kBlock) : zero8();
    float swv = 0.f;
    if constexpr (!kInt8) swv = sw[(n0 >> 7) * KB + kb];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const v8i af = avalid[mt] ? load32(ap[mt] + kb * kBlock) : zero8();
      if constexpr (kInt8) {
        acci[mt] = mfma_i8x2(wcur, af, acci[mt]);
      } else {
        const v4f p = mfma_fp8(wcur, af);
        const float s = (avalid[mt] ? sa[(mt * 16 + r16) * KB + kb] : 0.f) * swv;
#pragma unroll
        for (int r = 0; r < 4; ++r) accf[mt][r] = fmaf(p[r], s, accf[mt][r]);
      }
    }
  }

  // Cross-wave reduction of the K-split partial sums (int32 partials are
  // stored bit-cast in the same array).
  __shared__ float red[4][MT][4][64];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      red[wave][mt][r][lane] = kInt8 ? __int_as_float(acci[mt][r]) : accf[mt][r];
  __syncthreads();
  // Wave w finishes m-tiles w, w+4, ...
  for (int mt = wave; mt < MT; mt += 4) {
    const int64_t m = mt * 16 + r16;
    const int64_t n = n0 + 4 * g;
    float v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (kInt8) {
        const int32_t t = __float_as_int(red[0][mt][r][lane]) + __float_as_int(red[1][mt][r][lane]) +
                          __float_as_int(red[2][mt][r][lane]) + __float_as_int(red[3][mt][r][lane]);
        const float sm = (m < M) ? sa[m] : 0.f;
        const float sn = (n + r < N) ? sw[n + r] : 0.f;
        v[r] = (float)t * (sm * sn);
      } else {
        v[r] = (red[0][mt][r][lane] + red[1][mt][r][lane]) +
               (red[2][mt][r][lane] + red[3][mt][r][lane]);
      }
    }
    store4(C, M, N, m, n, v);
  }
}

// ---------------------------------------------------------------------------
// Tiled path (prefill / log-prob forward: M > 128).  A workgroup of 4 waves
// computes a 128 (n) x 128 (m) output tile; per 128-deep K block it stages
// the weight and activation tiles (16 KB each) through LDS, each wave then
// runs a 4 x 4 grid of 16 x 16 MFMA tiles on its 64 x 64 quarter.  LDS rows
// are 128 bytes; 16-byte chunk c of row r is stored at chunk c ^ (r mod 8)
// so that the 16 rows read together spread over the banks.
// ---------------------------------------------------------------------------
template <bool kInt8>
__global__ __launch_bounds__(256) void gemm_tile_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, int64_t M, int64_t N, int64_t K, uint16_t* __restrict__ C,
    int ntn) {
  __shared__ __align__(16) uint8_t lw[128 * 128];
  __shared__ __align__(16) uint8_t la[128 * 128];
  __shared__ float lsa[128];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const int wn = wave & 1, wm = wave >> 1;
  const int tn = blockIdx.x % ntn, tm = blockIdx.x / ntn;
  const int64_t n0 = (int64_t)tn * 128, m0 = (int64_t)tm * 128;
  const int64_t KB = K / kBlock;

  float accf[4][4][4];
  v4i acci[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acci[i][j] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[i][j][r] = 0.f;
    }

  for (int64_t kb = 0; kb < KB; ++kb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = i * 256 + tid;
      const int row = c >> 3, cc = c & 7;
      const int off = row * 128 + ((cc ^ (row & 7)) << 4);
      const int64_t wr = n0 + row, ar = m0 + row;
      const uint4 zw = make_uint4(0, 0, 0, 0);
      *reinterpret_cast<uint4*>(lw + off) =
          (wr < N) ? *reinterpret_cast<const uint4*>(W + wr * K + kb * kBlock + cc * 16) : zw;
      *reinterpret_cast<uint4*>(la + off) =
          (ar < M) ? *reinterpret_cast<const uint4*>(A + ar * K + kb * kBlock + cc * 16) : zw;
    }
    if constexpr (!kInt8) {
      if (tid < 128) lsa[tid] = (m0 + tid < M) ? sa[(m0 + tid) * KB + kb] : 0.f;
    }
    __syncthreads();

    v8i wf[4], af[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int rw = wn * 64 + t * 16 + r16;
      const int ra = wm * 64 + t * 16 + r16;
      const uint4 w0 = *reinterpret_cast<const uint4*>(lw + rw * 128 + (((2 * g) ^ (rw & 7)) << 4));
      const uint4 w1 = *reinterpret_cast<const uint4*>(lw + rw * 128 + (((2 * g + 1) ^ (rw & 7)) << 4));
      const uint4 a0 = *reinterpret_cast<const uint4*>(la + ra * 128 + (((2 * g) ^ (ra & 7)) << 4));
      const uint4 a1 = *reinterpret_cast<const uint4*>(la + ra * 128 + (((2 * g + 1) ^ (ra & 7)) << 4));
      wf[t] = v8i{(int)w0.x, (int)w0.y, (int)w0.z, (int)w0.w, (int)w1.x, (int)w1.y, (int)w1.z, (int)w1.w};
      af[t] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
    if constexpr (kInt8) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acci[i][j] = mfma_i8x2(wf[i], af[j], acci[i][j]);
    } else {
      const float swv = sw[(n0 >> 7) * KB + kb];
      float s[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = lsa[wm * 64 + j * 16 + r16] * swv;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const v4f p = mfma_fp8(wf[i], af[j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) accf[i][j][r] = fmaf(p[r], s[j], accf[i][j][r]);
        }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t m = m0 + wm * 64 + j * 16 + r16;
      const int64_t n = n0 + wn * 64 + i * 16 + 4 * g;
      float v[4];
      if constexpr (kInt8) {
        const float sm = (m < M) ? sa[m] : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (float)acci[i][j][r] * (sm * ((n + r < N) ? sw[n + r] : 0.f));
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = accf[i][j][r];
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
  if (M <= 128) {
    const unsigned grid = (unsigned)((N + 15) / 16);
    const int mt = (int)((M + 15) / 16);
#define PRR_SKINNY(T)                                                                          \
  case T:                                                                                      \
    hipLaunchKernelGGL((gemm_skinny_kernel<T, kInt8>), dim3(grid), dim3(256), 0, stream, A, sa, \
                       W, sw, M, N, K, C);                                                     \
    break;
    switch (mt) {
      PRR_SKINNY(1)
      PRR_SKINNY(2)
      PRR_SKINNY(3)
      PRR_SKINNY(4)
      PRR_SKINNY(5)
      PRR_SKINNY(6)
      PRR_SKINNY(7)
      PRR_SKINNY(8)
      default:
        return hipErrorInvalidValue;
    }
#undef PRR_SKINNY
    return hipGetLastError();
  }
  const int64_t ntn = (N + 127) / 128, ntm = (M + 127) / 128;
  hipLaunchKernelGGL((gemm_tile_kernel<kInt8>), dim3((unsigned)(ntn * ntm)), dim3(256), 0, stream,
                     A, sa, W, sw, M, N, K, C, (int)ntn);
  return hipGetLastError();
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

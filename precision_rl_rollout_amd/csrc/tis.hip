// Token-level importance weights for rollout correction ("FP8-RL: A
// Practical and Stable Low-Precision Stack for LLM Reinforcement Learning",
// abstract, item (iii): importance-sampling correction of the rollout /
// trainer mismatch at token level, truncated (TIS) or masked (MIS)).  Per
// response token: d = fl32(lp_train - lp_rollout); over = d > fl32(ln C);
// w = over ? (TIS: C, MIS: 0) : expf(d); padding tokens get w = 0.  Per
// sequence: valid tokens, tokens over the cap, sum of w, sum of
// lp_rollout - lp_train.  Bound by HBM: 13 bytes per token position (two
// fp32 log-probabilities and the mask read, the fp32 weight written).
#include "launch.h"
#include "prr_device.h"

namespace prr {

constexpr int kTisThreads = 256;
constexpr int kTisUnroll = 4;       // 4-token chunks in flight per thread

struct TisPartial {
  int n_valid = 0, n_over = 0;
  float sum_w = 0.f, sum_kl = 0.f;
};

__device__ __forceinline__ float tis_token(float lt, float lr, bool valid, float cap, float lncap,
                                           int mode, TisPartial& p) {
  const float d = __fsub_rn(lt, lr);
  const bool over = valid && d > lncap;
  const float rho = expf(d);
  float w = over ? (mode == 0 ? cap : 0.f) : rho;
  w = valid ? w : 0.f;
  p.n_valid += valid ? 1 : 0;
  p.n_over += over ? 1 : 0;
  p.sum_w += w;
  p.sum_kl += valid ? -d : 0.f;
  return w;
}

// One workgroup per sequence.  Vector path (T % 4 == 0): thread i takes the
// 4-token chunks i, i + 256, ... of its row, kTisUnroll of them per pass with
// every load issued before the first use.
template <bool kVec>
__global__ __launch_bounds__(kTisThreads) void tis_row_kernel(
    const float* __restrict__ lp_train, const float* __restrict__ lp_rollout,
    const uint8_t* __restrict__ mask, int64_t T, float cap, float lncap, int mode,
    float* __restrict__ w, float* __restrict__ row_stats) {
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  const float* lt = lp_train + b * T;
  const float* lr = lp_rollout + b * T;
  const uint8_t* mk = mask + b * T;
  float* wo = w + b * T;
  TisPartial p;
  if constexpr (kVec) {
    const int64_t chunks = T / 4;
    for (int64_t c0 = tid; c0 < chunks; c0 += (int64_t)kTisThreads * kTisUnroll) {
      float4 a[kTisUnroll], r[kTisUnroll];
      uint32_t m[kTisUnroll];
#pragma unroll
      for (int u = 0; u < kTisUnroll; ++u) {
        const int64_t c = c0 + (int64_t)u * kTisThreads;
        const bool in = c < chunks;
        const uint4 x = in ? load_once16(lt + 4 * c) : make_uint4(0, 0, 0, 0);
        const uint4 y = in ? load_once16(lr + 4 * c) : make_uint4(0, 0, 0, 0);
        a[u] = make_float4(__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                           __uint_as_float(x.w));
        r[u] = make_float4(__uint_as_float(y.x), __uint_as_float(y.y), __uint_as_float(y.z),
                           __uint_as_float(y.w));
        m[u] = in ? __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(mk) + c) : 0u;
      }
#pragma unroll
      for (int u = 0; u < kTisUnroll; ++u) {
        const int64_t c = c0 + (int64_t)u * kTisThreads;
        if (c >= chunks) break;
        float4 o;
        o.x = tis_token(a[u].x, r[u].x, (m[u] & 0xFFu) != 0, cap, lncap, mode, p);
        o.y = tis_token(a[u].y, r[u].y, (m[u] & 0xFF00u) != 0, cap, lncap, mode, p);
        o.z = tis_token(a[u].z, r[u].z, (m[u] & 0xFF0000u) != 0, cap, lncap, mode, p);
        o.w = tis_token(a[u].w, r[u].w, (m[u] & 0xFF000000u) != 0, cap, lncap, mode, p);
        reinterpret_cast<float4*>(wo)[c] = o;
      }
    }
  } else {
    for (int64_t t = tid; t < T; t += kTisThreads)
      wo[t] = tis_token(lt[t], lr[t], mk[t] != 0, cap, lncap, mode, p);
  }
  if (row_stats == nullptr) return;
  // Fixed-order reduction: butterfly within each wave, then the 4 wave
  // results added in wave order.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    p.n_valid += __shfl_xor(p.n_valid, off, 64);
    p.n_over += __shfl_xor(p.n_over, off, 64);
    p.sum_w += __shfl_xor(p.sum_w, off, 64);
    p.sum_kl += __shfl_xor(p.sum_kl, off, 64);
  }
  __shared__ float part[kTisThreads / 64][4];
  if ((tid & 63) == 0) {
    part[tid >> 6][0] = (float)p.n_valid;        // exact: T <= 2^24
    part[tid >> 6][1] = (float)p.n_over;
    part[tid >> 6][2] = p.sum_w;
    part[tid >> 6][3] = p.sum_kl;
  }
  __syncthreads();
  if (tid < 4) {
    float s = 0.f;
    if (tid < 2) {
      int n = 0;
#pragma unroll
      for (int q = 0; q < kTisThreads / 64; ++q) n += (int)part[q][tid];
      s = (float)n;
    } else {
#pragma unroll
      for (int q = 0; q < kTisThreads / 64; ++q) s += part[q][tid];
    }
    row_stats[b * 4 + tid] = s;
  }
}

// Batch totals from the row statistics: one workgroup, fp64, fixed order
// (thread i adds rows i, i + 256, ... in order, then a butterfly and the
// 4 wave results in wave order).  A thread's rows are loaded kTotalRows at a
// time (16 bytes each, all issued before the first add).  B == 0 writes
// zeros.
constexpr int kTotalRows = 8;

__global__ __launch_bounds__(kTisThreads) void tis_total_kernel(const float* __restrict__ row_stats,
                                                                int64_t B,
                                                                double* __restrict__ totals) {
  const int tid = threadIdx.x;
  double s[4] = {0.0, 0.0, 0.0, 0.0};
  for (int64_t b0 = tid; b0 < B; b0 += (int64_t)kTisThreads * kTotalRows) {
    float4 v[kTotalRows];
#pragma unroll
    for (int u = 0; u < kTotalRows; ++u) {
      const int64_t b = b0 + (int64_t)u * kTisThreads;
      v[u] = b < B ? reinterpret_cast<const float4*>(row_stats)[b] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kTotalRows; ++u) {
      s[0] += (double)v[u].x;
      s[1] += (double)v[u].y;
      s[2] += (double)v[u].z;
      s[3] += (double)v[u].w;
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] += __shfl_xor(s[j], off, 64);
  __shared__ double part[kTisThreads / 64][4];
  if ((tid & 63) == 0)
#pragma unroll
    for (int j = 0; j < 4; ++j) part[tid >> 6][j] = s[j];
  __syncthreads();
  if (tid < 4) {
    double t = 0.0;
#pragma unroll
    for (int q = 0; q < kTisThreads / 64; ++q) t += part[q][tid];
    totals[tid] = t;
  }
}

hipError_t launch_tis_token_weights(const float* lp_train, const float* lp_rollout,
                                    const uint8_t* mask, int64_t B, int64_t T, float cap,
                                    float lncap, int mode, float* w, float* row_stats,
                                    double* totals, hipStream_t stream) {
  if (B > 0) {
    if (T % 4 == 0)
      hipLaunchKernelGGL(tis_row_kernel<true>, dim3((unsigned)B), dim3(kTisThreads), 0, stream,
                         lp_train, lp_rollout, mask, T, cap, lncap, mode, w, row_stats);
    else
      hipLaunchKernelGGL(tis_row_kernel<false>, dim3((unsigned)B), dim3(kTisThreads), 0, stream,
                         lp_train, lp_rollout, mask, T, cap, lncap, mode, w, row_stats);
  }
  if (totals != nullptr)
    hipLaunchKernelGGL(tis_total_kernel, dim3(1), dim3(kTisThreads), 0, stream, row_stats, B,
                       totals);
  return hipGetLastError();
}

}  // namespace prr

// FP8 KV cache: per-step scale recalibration and quantize-on-write
// ("FP8-RL: A Practical and Stable Low-Precision Stack for LLM Reinforcement
// Learning", abstract, item (ii): FP8 KV cache with per-step QKV scale
// recalibration).  One scale per tensor, s = fl32(amax / 448), and the same
// saturating round-to-nearest-even e4m3 encode of fl32(x / s) as the weight
// and activation quantizers.  Both kernels are bound by HBM: 2 bytes read
// per element for the recalibration, 2 read + 1 written for the write.
#include "launch.h"
#include "prr_device.h"

namespace prr {

// Each workgroup turns its own amax into a scale, fl32(amax_wg / 448), and
// folds it into the caller's scale word with an integer atomic maximum: the
// bit order of non-negative floats is their value order, and a correctly
// rounded division by a positive constant is monotone, so the maximum of the
// workgroups' scales is fl32(amax / 448) of the whole tensor, whatever the
// order of the updates.  No kernel runs after the reduction.
__global__ void kv_amax_clear_kernel(uint32_t* acc) { *acc = 0u; }

// Each thread takes kAmaxLoads 16-byte chunks per pass, all loads issued
// before any is used (one load in flight per thread held it to ~1.9 TB/s).
// The grid is at most one workgroup per CU, looping over the passes: the
// atomics of more workgroups, all ending together, serialize on the one
// word (at 131,072 x 1024 values, 1024 workgroups took 65 us, 256 took 47).
constexpr int kAmaxLoads = 32;

__global__ __launch_bounds__(256) void kv_amax_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                      uint32_t* __restrict__ acc) {
  __shared__ uint32_t red[4];
  const int tid = threadIdx.x;
  const int64_t chunks = n / 8;
  const int64_t stride = (int64_t)gridDim.x * 256;
  uint32_t m = 0;
  for (int64_t c0 = (int64_t)blockIdx.x * 256 + tid; c0 < chunks; c0 += stride * kAmaxLoads) {
    uint4 v[kAmaxLoads];
#pragma unroll
    for (int u = 0; u < kAmaxLoads; ++u) {
      const int64_t c = c0 + u * stride;
      v[u] = c < chunks ? load_once16(x + c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kAmaxLoads; ++u) {
      m = absmax_bf16x2(m, v[u].x);
      m = absmax_bf16x2(m, v[u].y);
      m = absmax_bf16x2(m, v[u].z);
      m = absmax_bf16x2(m, v[u].w);
    }
  }
  m = absmax_fold(m);
  if (blockIdx.x == 0) {
    for (int64_t e = chunks * 8 + tid; e < n; e += 256) m = max(m, (uint32_t)(x[e] & 0x7FFFu));
  }
  m = wave_max_u32(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  if (tid == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    if (m) atomicMax(acc, __float_as_uint(div_rn(__uint_as_float(m << 16), kFp8Max)));
  }
}

hipError_t launch_fp8_kv_scale_recalibrate(const uint16_t* x, int64_t n, float* scale,
                                           hipStream_t stream) {
  uint32_t* acc = reinterpret_cast<uint32_t*>(scale);
  hipLaunchKernelGGL(kv_amax_clear_kernel, dim3(1), dim3(1), 0, stream, acc);
  if (n > 0) {
    const int64_t chunks = n / 8;
    int64_t grid = (chunks + 256 * kAmaxLoads - 1) / (256 * kAmaxLoads);
    const int64_t cap = compute_units();
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(kv_amax_kernel, dim3((unsigned)grid), dim3(256), 0, stream, x, n, acc);
  }
  return hipGetLastError();
}

// Quantize-on-write.  A workgroup of 256 threads covers `rpw` token rows of
// C values with lpr = 256 / rpw threads per row; a thread takes up to
// kWriteChunks 16-byte chunks of its row (8 values each; chunk i of the
// thread is chunk lane + i * lpr of the row), issuing every load before the
// first encode, and the slot lookup after them, so the loads overlap.  Rows
// whose slot is outside [0, num_slots) are skipped.  The scale comes from an
// earlier batch, so quotients are not bounded by 448 and are clamped before
// the conversion.
constexpr int kWriteChunks = 4;

// kRecal (fp8_kv_cache_write_recalibrate): the same pass also reduces the
// rows' amax -- over every row of the batch, whether or not its slot is in
// range -- and each workgroup stores its packed maximum in part[blockIdx.x]
// with a plain store; kv_part_scale_kernel then folds the partials into the
// new scale.  (One atomic maximum per workgroup on the single scale word
// serializes on that word: at 2048 workgroups it added ~9 us to a 12 us
// write; spread over 64 words it added nothing.)  The grid is capped at
// kKvRecalParts workgroups, which loop over the row groups, so the partials
// fit the caller's fixed workspace.  No thread leaves before the
// workgroup's reduction: rows past T and rows with no slot only skip their
// stores.
template <bool kVec, bool kRecal>
__device__ __forceinline__ void kv_write_rows(
    const uint16_t* __restrict__ kv, const int64_t* __restrict__ slots, int64_t T, int64_t C,
    const float* __restrict__ scale, uint8_t* __restrict__ cache, int64_t num_slots, int rpw,
    uint32_t* __restrict__ part) {
  const int lpr = 256 / rpw;                      // threads per row
  const int64_t lane8 = (int64_t)(threadIdx.x % lpr) * 8;
  const int64_t step = (int64_t)lpr * 8;
  const int64_t groups = (T + rpw - 1) / rpw;
  uint32_t am = 0;                                // packed |x| maxima (kRecal)
  // One row group per workgroup for the plain write; a grid-stride loop
  // over them for kRecal.
  for (int64_t g = blockIdx.x; g < groups; g += kRecal ? (int64_t)gridDim.x : groups) {
    const int64_t t = g * rpw + threadIdx.x / lpr;
    const bool row_live = t < T;
    if (!kRecal && !row_live) return;
    const uint16_t* src = kv + (row_live ? t : 0) * C;
    for (int64_t col0 = lane8; col0 < C; col0 += step * kWriteChunks) {
      uint4 v[kWriteChunks];
#pragma unroll
      for (int i = 0; i < kWriteChunks; ++i) {
        const int64_t col = col0 + i * step;
        const bool in = row_live && col < C;
        if constexpr (kVec) {       // C % 8 == 0: whole 16-byte chunks, aligned
          v[i] = in ? load_once16(src + col) : make_uint4(0, 0, 0, 0);
        } else {
          uint32_t h[8];
#pragma unroll
          for (int e = 0; e < 8; ++e)
            h[e] = (row_live && col + e < C) ? (uint32_t)src[col + e] : 0u;
          v[i] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                            h[6] | (h[7] << 16));
        }
      }
      if constexpr (kRecal) {
#pragma unroll
        for (int i = 0; i < kWriteChunks; ++i) {
          am = absmax_bf16x2(am, v[i].x);
          am = absmax_bf16x2(am, v[i].y);
          am = absmax_bf16x2(am, v[i].z);
          am = absmax_bf16x2(am, v[i].w);
        }
      }
      const int64_t slot = row_live ? slots[t] : -1;
      if (slot < 0 || slot >= num_slots) {
        if constexpr (kRecal) continue;
        else return;
      }
      const float s = *scale;
      const BlockDiv d = block_div(s);
      uint8_t* dst = cache + slot * C;
#pragma unroll
      for (int i = 0; i < kWriteChunks; ++i) {
        const int64_t col = col0 + i * step;
        if (col >= C) break;
        const uint2 c = e4m3_chunk_any<true>(v[i], s, d);
        if constexpr (kVec) {
          *reinterpret_cast<uint2*>(dst + col) = c;
        } else {
          const uint32_t cw[2] = {c.x, c.y};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (col + e < C) dst[col + e] = (uint8_t)(cw[e >> 2] >> (8 * (e & 3)));
        }
      }
    }
  }
  if constexpr (kRecal) {
    __shared__ uint32_t red[4];
    uint32_t m = wave_max_u32(absmax_fold(am));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) part[blockIdx.x] = max(max(red[0], red[1]), max(red[2], red[3]));
  }
}

template <bool kVec>
__global__ __launch_bounds__(256) void kv_cache_write_kernel(
    const uint16_t* __restrict__ kv, const int64_t* __restrict__ slots, int64_t T, int64_t C,
    const float* __restrict__ scale, uint8_t* __restrict__ cache, int64_t num_slots, int rpw) {
  kv_write_rows<kVec, false>(kv, slots, T, C, scale, cache, num_slots, rpw, nullptr);
}

// The write with recalibration for several tensors sharing the slot mapping
// (K and V of a step): workgroup (x, j) works on job j, its partials at
// part + j kKvRecalParts.
template <bool kVec>
__global__ __launch_bounds__(256) void kv_cache_write_recal_kernel(
    KvJobs jobs, const int64_t* __restrict__ slots, int64_t T, int64_t C, int64_t num_slots,
    int rpw, uint32_t* __restrict__ part) {
  const int j = blockIdx.y;
  kv_write_rows<kVec, true>(jobs.kv[j], slots, T, C, jobs.scale[j], jobs.cache[j], num_slots,
                            rpw, part + (int64_t)j * kKvRecalParts);
}

// The new scale of job blockIdx.x from its n partial maxima: fl32(amax /
// 448), +0.0 when every partial is 0 (an all-zero or empty batch).  One
// workgroup per job.  Its trace duration, ~4 us, is the kernel boundary
// (the same as the one-thread clear kernel's after a large write): two
// 16-byte loads per thread instead of this loop measured the same.
__global__ __launch_bounds__(256) void kv_part_scale_kernel(KvJobs jobs,
                                                            const uint32_t* __restrict__ part,
                                                            int n) {
  __shared__ uint32_t red[4];
  const uint32_t* pj = part + (int64_t)blockIdx.x * kKvRecalParts;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += 256) m = max(m, pj[i]);
  m = wave_max_u32(m);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = max(max(red[0], red[1]), max(red[2], red[3]));
    *jobs.new_scale[blockIdx.x] = m ? div_rn(__uint_as_float(m << 16), kFp8Max) : 0.0f;
  }
}

static int kv_rows_per_wg(int64_t C) {
  // Threads per row: enough for kWriteChunks chunks each (at most 256).
  const int64_t chunks = (C + 7) / 8;
  const int64_t per = (chunks + kWriteChunks - 1) / kWriteChunks;
  int rpw = 1;                                    // rows per workgroup
  while (rpw < 256 && 256 / (rpw * 2) >= per) rpw *= 2;
  return rpw;
}

hipError_t launch_fp8_kv_cache_write(const uint16_t* kv, const int64_t* slots, int64_t T,
                                     int64_t C, const float* scale, uint8_t* cache,
                                     int64_t num_slots, hipStream_t stream) {
  const int rpw = kv_rows_per_wg(C);
  const unsigned grid = (unsigned)((T + rpw - 1) / rpw);
  if (C % 8 == 0)
    hipLaunchKernelGGL(kv_cache_write_kernel<true>, dim3(grid), dim3(256), 0, stream, kv, slots,
                       T, C, scale, cache, num_slots, rpw);
  else
    hipLaunchKernelGGL(kv_cache_write_kernel<false>, dim3(grid), dim3(256), 0, stream, kv,
                       slots, T, C, scale, cache, num_slots, rpw);
  return hipGetLastError();
}

hipError_t launch_fp8_kv_cache_write_recalibrate(const KvJobs& jobs, const int64_t* slots,
                                                 int64_t T, int64_t C, int64_t num_slots,
                                                 uint32_t* part, hipStream_t stream) {
  if (jobs.count < 1) return hipSuccess;
  int grid = 0;
  if (T > 0 && C > 0) {
    const int rpw = kv_rows_per_wg(C);
    const int64_t groups = (T + rpw - 1) / rpw;
    grid = (int)(groups < kKvRecalParts ? groups : kKvRecalParts);
    const dim3 g((unsigned)grid, (unsigned)jobs.count);
    if (C % 8 == 0)
      hipLaunchKernelGGL(kv_cache_write_recal_kernel<true>, g, dim3(256), 0, stream, jobs, slots,
                         T, C, num_slots, rpw, part);
    else
      hipLaunchKernelGGL(kv_cache_write_recal_kernel<false>, g, dim3(256), 0, stream, jobs,
                         slots, T, C, num_slots, rpw, part);
  }
  hipLaunchKernelGGL(kv_part_scale_kernel, dim3((unsigned)jobs.count), dim3(256), 0, stream, jobs,
                     part, grid);
  return hipGetLastError();
}

}  // namespace prr

// INT8 re-quantization kernels: one fp32 scale amax / 127 per weight row
// (output channel) or per activation row (token) over the whole K (FlashRL
// article: INT8 rollout with the weights re-quantized after every update;
// the granularity is fixed by this library).
//
// A row is held in registers between its amax reduction and the encode, so
// every element is read from HBM once:
//   * K <= 8192:  one wave per row (up to 16 x 16-byte chunks per lane),
//                 4 rows per 256-thread workgroup, reduction inside the wave;
//   * K <= 32768: one 256-thread workgroup per row, reduction through LDS;
//   * longer rows (and K % 8 != 0): a workgroup per row reads the row twice,
//                 the second time from the L2 the first pass filled.
#include "launch.h"
#include "prr_device.h"

namespace prr {

constexpr int kMaxChunks = 16;       // 16-byte chunks a lane keeps in registers

template <int kClass>
__device__ __forceinline__ uint2 int8_chunk_class(uint4 w, const BlockDiv& d) {
  if constexpr (kClass == 0) return make_uint2(0u, 0u);
  else return int8_chunk<kClass == 2>(w, d);
}

template <int kClass, int kLanes, bool kStream>
__device__ __forceinline__ void int8_store_row(const uint4 (&v)[kMaxChunks], const BlockDiv& d,
                                               uint8_t* __restrict__ dst, int64_t chunks,
                                               int lane) {
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int64_t c = (int64_t)i * kLanes + lane;
    if (c < chunks) store_codes8<kStream>(dst + c * 8, int8_chunk_class<kClass>(v[i], d));
  }
}

// Register-resident row: kLanes lanes (64: a wave, 256: the workgroup) per
// row; work unit u is rows 256 / kLanes u ...  Called by all 256 threads.
// kStream: non-temporal code stores (store_codes8).
template <int kLanes, bool kStream>
__device__ __forceinline__ void int8_rows_resident(const uint16_t* __restrict__ x, int64_t R,
                                                   int64_t K, int8_t* __restrict__ q,
                                                   float* __restrict__ scale, int64_t unit) {
  constexpr int kRowsPerWg = 256 / kLanes;
  const int tid = threadIdx.x;
  const int lane = tid % kLanes;
  const int64_t row = unit * kRowsPerWg + tid / kLanes;
  const bool live = row < R;                    // uniform per row group
  const int64_t chunks = K / 8;
  const uint16_t* src = x + row * K;
  uint4 v[kMaxChunks];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < kMaxChunks; ++i) {
    const int64_t c = (int64_t)i * kLanes + lane;
    v[i] = (live && c < chunks) ? load_once16(src + c * 8)
                                : make_uint4(0, 0, 0, 0);
    m = absmax_bf16x2(m, v[i].x);
    m = absmax_bf16x2(m, v[i].y);
    m = absmax_bf16x2(m, v[i].z);
    m = absmax_bf16x2(m, v[i].w);
  }
  m = wave_max_u32(absmax_fold(m));
  if constexpr (kLanes == 256) {
    __shared__ uint32_t red[4];
    if ((tid & 63) == 0) red[tid >> 6] = m;
    __syncthreads();
    m = max(max(red[0], red[1]), max(red[2], red[3]));
  }
  if (!live) return;
  const float s = div_rn(__uint_as_float(m << 16), kInt8Max);
  if (lane == 0) scale[row] = s;
  const BlockDiv d = block_div(s);
  uint8_t* dst = reinterpret_cast<uint8_t*>(q) + row * K;
  if (s == 0.0f) int8_store_row<0, kLanes, kStream>(v, d, dst, chunks, lane);
  else if (d.tiny) int8_store_row<2, kLanes, kStream>(v, d, dst, chunks, lane);
  else int8_store_row<1, kLanes, kStream>(v, d, dst, chunks, lane);
}

template <int kLanes>
__global__ __launch_bounds__(256) void int8_row_resident_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t K, int8_t* __restrict__ q,
    float* __restrict__ scale) {
  int8_rows_resident<kLanes, false>(x, R, K, q, scale, blockIdx.x);
}

// Any K: a workgroup per row, two passes; 16-byte chunks when K % 8 == 0,
// single elements otherwise.  Called by all 256 threads.
template <bool kStream>
__device__ __forceinline__ void int8_row_twopass(const uint16_t* __restrict__ x, int64_t K,
                                                 int8_t* __restrict__ q,
                                                 float* __restrict__ scale, int64_t row) {
  __shared__ uint32_t red[4];
  const uint16_t* src = x + row * K;
  uint8_t* dst = reinterpret_cast<uint8_t*>(q) + row * K;
  const int tid = threadIdx.x;
  const bool vec = (K % 8) == 0;
  uint32_t m = 0;
  if (vec) {
    for (int64_t c = tid; c < K / 8; c += 256) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c * 8);
      m = absmax_bf16x2(m, v.x);
      m = absmax_bf16x2(m, v.y);
      m = absmax_bf16x2(m, v.z);
      m = absmax_bf16x2(m, v.w);
    }
    m = absmax_fold(m);
  } else {
    for (int64_t k = tid; k < K; k += 256) m = max(m, (uint32_t)(src[k] & 0x7FFFu));
  }
  m = wave_max_u32(m);
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  const float s = div_rn(__uint_as_float(m << 16), kInt8Max);
  if (tid == 0) scale[row] = s;
  const BlockDiv d = block_div(s);
  if (vec) {
    for (int64_t c = tid; c < K / 8; c += 256) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c * 8);
      store_codes8<kStream>(dst + c * 8, int8_chunk_any(v, s, d));
    }
  } else {
    for (int64_t k = tid; k < K; k += 256) {
      const float xv = __uint_as_float((uint32_t)src[k] << 16);
      uint32_t c = 0;
      if (s != 0.0f) c = int8_code(d.tiny ? div_block<true>(xv, d) : div_block<false>(xv, d));
      dst[k] = (uint8_t)c;
    }
  }
}

__global__ __launch_bounds__(256) void int8_row_twopass_kernel(
    const uint16_t* __restrict__ x, int64_t K, int8_t* __restrict__ q,
    float* __restrict__ scale) {
  int8_row_twopass<false>(x, K, q, scale, blockIdx.x);
}

// Row classes: 0 = a wave per row (4 rows per work unit), 1 = a workgroup
// per row held in registers, 2 = two passes.
int int8_row_class(int64_t K) {
  if (K % 8 == 0 && K <= 64 * 8 * kMaxChunks) return 0;
  if (K % 8 == 0 && K <= 256 * 8 * kMaxChunks) return 1;
  return 2;
}

int int8_rows_per_unit(int cls) { return cls == 0 ? 4 : 1; }

// Several weights in one grid, as the FP8 multi-weight kernel: workgroup b
// takes work unit b of the job whose range holds it; the job's row class is
// uniform, so each workgroup runs one of the three row paths.  Codes are
// stored non-temporal, as in the FP8 multi-weight kernel.
__global__ __launch_bounds__(256) void int8_row_multi_kernel(WeightJobs jobs) {
  const int b = blockIdx.x;
  int j = 0;
#pragma unroll 1
  while (j + 1 < jobs.count && b >= jobs.first[j + 1]) ++j;
  j = __builtin_amdgcn_readfirstlane(j);
  const int64_t unit = b - jobs.first[j];
  const int cls = jobs.units_per_row[j];
  int8_t* q = static_cast<int8_t*>(jobs.q[j]);
  if (cls == 0)
    int8_rows_resident<64, true>(jobs.w[j], jobs.N[j], jobs.K[j], q, jobs.scale[j], unit);
  else if (cls == 1)
    int8_rows_resident<256, true>(jobs.w[j], jobs.N[j], jobs.K[j], q, jobs.scale[j], unit);
  else
    int8_row_twopass<true>(jobs.w[j], jobs.K[j], q, jobs.scale[j], unit);
}

hipError_t launch_int8_weight_channel_quant_multi(const WeightJobs& jobs, hipStream_t stream) {
  const int units = jobs.first[jobs.count];
  if (units > 0)
    hipLaunchKernelGGL(int8_row_multi_kernel, dim3((unsigned)units), dim3(256), 0, stream, jobs);
  return hipGetLastError();
}

static hipError_t launch_int8_rows(const uint16_t* x, int64_t R, int64_t K, int8_t* q,
                                   float* scale, hipStream_t stream) {
  const int cls = int8_row_class(K);
  if (cls == 0)
    hipLaunchKernelGGL(int8_row_resident_kernel<64>, dim3((unsigned)((R + 3) / 4)), dim3(256), 0,
                       stream, x, R, K, q, scale);
  else if (cls == 1)
    hipLaunchKernelGGL(int8_row_resident_kernel<256>, dim3((unsigned)R), dim3(256), 0, stream, x,
                       R, K, q, scale);
  else
    hipLaunchKernelGGL(int8_row_twopass_kernel, dim3((unsigned)R), dim3(256), 0, stream, x, K, q,
                       scale);
  return hipGetLastError();
}

hipError_t launch_int8_weight_channel_quant(const uint16_t* w, int64_t N, int64_t K, int8_t* q,
                                            float* scale, hipStream_t stream) {
  return launch_int8_rows(w, N, K, q, scale, stream);
}

hipError_t launch_int8_act_token_quant(const uint16_t* a, int64_t M, int64_t K, int8_t* q,
                                       float* scale, hipStream_t stream) {
  return launch_int8_rows(a, M, K, q, scale, stream);
}

}  // namespace prr

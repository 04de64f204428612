// INT8 re-quantization kernels: one fp32 scale amax / 127 per weight row
// (output channel) or per activation row (token) over the whole K (FlashRL
// article: INT8 rollout with the weights re-quantized after every update;
// the granularity is fixed by this library).
//
// One 256-thread workgroup per row.  Rows up to kResident elements stay in
// registers between the amax reduction and the encode, so every element is
// read from HBM once; longer rows are read twice, the second time from the
// L2 that the first pass just filled.
#include "launch.h"
#include "prr_device.h"

namespace prr {

constexpr int kRowThreads = 256;
constexpr int kResidentChunks = 8;                           // 16-byte chunks per lane
constexpr int64_t kResident = kRowThreads * 8 * kResidentChunks;  // 16384 elements

__device__ __forceinline__ float block_amax(uint32_t m, uint32_t* red) {
  m = wave_max_u32(m);
  const int tid = threadIdx.x;
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  return __uint_as_float(m << 16);
}

// K % 8 == 0: 16-byte chunks.
template <bool kResidentRow>
__global__ __launch_bounds__(kRowThreads) void int8_row_kernel_vec(
    const uint16_t* __restrict__ x, int64_t K, int8_t* __restrict__ q,
    float* __restrict__ scale) {
  __shared__ uint32_t red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* src = x + row * K;
  uint8_t* dst = reinterpret_cast<uint8_t*>(q) + row * K;
  const int64_t chunks = K / 8;
  const int tid = threadIdx.x;
  uint32_t m = 0;
  if constexpr (kResidentRow) {
    uint4 v[kResidentChunks];
#pragma unroll
    for (int i = 0; i < kResidentChunks; ++i) {
      const int64_t c = (int64_t)i * kRowThreads + tid;
      v[i] = (c < chunks) ? *reinterpret_cast<const uint4*>(src + c * 8) : make_uint4(0, 0, 0, 0);
      m = absmax_bf16x2(m, v[i].x);
      m = absmax_bf16x2(m, v[i].y);
      m = absmax_bf16x2(m, v[i].z);
      m = absmax_bf16x2(m, v[i].w);
    }
    const float s = div_rn(block_amax(m, red), kInt8Max);
    if (tid == 0) scale[row] = s;
#pragma unroll
    for (int i = 0; i < kResidentChunks; ++i) {
      const int64_t c = (int64_t)i * kRowThreads + tid;
      if (c < chunks) *reinterpret_cast<uint2*>(dst + c * 8) = int8_chunk(v[i], s);
    }
  } else {
    for (int64_t c = tid; c < chunks; c += kRowThreads) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c * 8);
      m = absmax_bf16x2(m, v.x);
      m = absmax_bf16x2(m, v.y);
      m = absmax_bf16x2(m, v.z);
      m = absmax_bf16x2(m, v.w);
    }
    const float s = div_rn(block_amax(m, red), kInt8Max);
    if (tid == 0) scale[row] = s;
    for (int64_t c = tid; c < chunks; c += kRowThreads) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c * 8);
      *reinterpret_cast<uint2*>(dst + c * 8) = int8_chunk(v, s);
    }
  }
}

// Any K: element-wise, bounds-checked.
__global__ __launch_bounds__(kRowThreads) void int8_row_kernel_any(
    const uint16_t* __restrict__ x, int64_t K, int8_t* __restrict__ q,
    float* __restrict__ scale) {
  __shared__ uint32_t red[4];
  const int64_t row = blockIdx.x;
  const uint16_t* src = x + row * K;
  const int tid = threadIdx.x;
  uint32_t m = 0;
  for (int64_t k = tid; k < K; k += kRowThreads) m = max(m, (uint32_t)(src[k] & 0x7FFFu));
  const float s = div_rn(block_amax(m, red), kInt8Max);
  if (tid == 0) scale[row] = s;
  for (int64_t k = tid; k < K; k += kRowThreads) {
    const float xv = __uint_as_float((uint32_t)src[k] << 16);
    q[row * K + k] = (int8_t)(s != 0.0f ? int8_code(div_rn(xv, s)) : 0u);
  }
}

static hipError_t launch_int8_rows(const uint16_t* x, int64_t R, int64_t K, int8_t* q,
                                   float* scale, hipStream_t stream) {
  if (K % 8 == 0 && K <= kResident)
    hipLaunchKernelGGL(int8_row_kernel_vec<true>, dim3((unsigned)R), dim3(kRowThreads), 0,
                       stream, x, K, q, scale);
  else if (K % 8 == 0)
    hipLaunchKernelGGL(int8_row_kernel_vec<false>, dim3((unsigned)R), dim3(kRowThreads), 0,
                       stream, x, K, q, scale);
  else
    hipLaunchKernelGGL(int8_row_kernel_any, dim3((unsigned)R), dim3(kRowThreads), 0, stream, x,
                       K, q, scale);
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

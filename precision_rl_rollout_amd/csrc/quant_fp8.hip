// FP8 e4m3 re-quantization kernels: 128 x 128 weight blocks and 1 x 128
// per-token activation groups, one fp32 scale amax / 448 per block or group
// (FP8-RL, abstract: weights change every step and are quantized again;
// item (i): blockwise FP8 W8A8).
//
// Both kernels read each bf16 element once from HBM, keep it in registers
// while the block's amax is reduced, and write one code byte per element
// plus one scale per block: 3 bytes of traffic per element.
#include "launch.h"
#include "prr_device.h"

namespace prr {

// ---------------------------------------------------------------------------
// Weight blocks.  One 256-thread workgroup per 128 x 128 block.  Each group
// of 16 lanes covers one 128-element row segment (16 lanes x 8 bf16 = 256
// bytes, a fully coalesced row); the workgroup walks 16 rows per step, 8
// steps, so every lane holds 64 bf16 in 8 x 16-byte registers.
// ---------------------------------------------------------------------------
// Encode the 8 chunks a lane holds and store them (block-uniform class:
// kClass 0 = all-zero block, 1 = ordinary, 2 = tiny scale; kStream:
// non-temporal code stores, see store_codes8).
template <int kClass, bool kStream>
__device__ __forceinline__ void encode_block_rows(const uint4 (&v)[8], const BlockDiv& d,
                                                  bool full, uint8_t* __restrict__ q, int64_t N,
                                                  int64_t K, int64_t ldq, int64_t row0, int seg,
                                                  int64_t col) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = row0 + i * 16 + seg;
    uint2 c;
    if constexpr (kClass == 0) c = e4m3_zero_chunk(v[i]);
    else c = e4m3_chunk<kClass == 2>(v[i], d);
    if (full) {
      store_codes8<kStream>(q + r * ldq + col, c);
    } else {
      const uint32_t cw[2] = {c.x, c.y};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (r < N && col + e < K) q[r * ldq + col + e] = (uint8_t)(cw[e >> 2] >> (8 * (e & 3)));
    }
  }
}

// Block (bi, bj) of an N x K matrix with row strides ldw (input, elements),
// ldq (codes, bytes) and lds (scales, floats); the whole-weight call has
// ldw = ldq = K and lds = nbk.  Called by all 256 threads of a workgroup.
template <bool kStream>
__device__ __forceinline__ void fp8_weight_block(const uint16_t* __restrict__ w, int64_t N,
                                                 int64_t K, int64_t ldw, uint8_t* __restrict__ q,
                                                 int64_t ldq, float* __restrict__ scale,
                                                 int64_t lds, int bi, int bj) {
  const int tid = threadIdx.x;
  const int seg = tid >> 4;       // row within a step, 0..15
  const int l16 = tid & 15;       // 8-element chunk within the row segment
  const int64_t row0 = (int64_t)bi * kBlock;
  const int64_t col = (int64_t)bj * kBlock + l16 * 8;
  // Workgroup-uniform: a complete block with 16-byte aligned input rows and
  // 8-byte aligned code rows takes the vector path; edge blocks of ragged
  // shapes take the bounds-checked one.
  const bool full = (row0 + kBlock <= N) && ((int64_t)(bj + 1) * kBlock <= K) &&
                    (ldw % 8 == 0) && (ldq % 8 == 0);

  uint4 v[8];
  if (full) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = row0 + i * 16 + seg;
      v[i] = load_once16(w + r * ldw + col);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = row0 + i * 16 + seg;
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        h[e] = (r < N && col + e < K) ? (uint32_t)w[r * ldw + col + e] : 0u;
      v[i] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                        h[6] | (h[7] << 16));
    }
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    m = absmax_bf16x2(m, v[i].x);
    m = absmax_bf16x2(m, v[i].y);
    m = absmax_bf16x2(m, v[i].z);
    m = absmax_bf16x2(m, v[i].w);
  }
  m = wave_max_u32(absmax_fold(m));
  __shared__ uint32_t red[4];
  if ((tid & 63) == 0) red[tid >> 6] = m;
  __syncthreads();
  m = max(max(red[0], red[1]), max(red[2], red[3]));
  const float amax = __uint_as_float(m << 16);
  const float s = div_rn(amax, kFp8Max);
  if (tid == 0) scale[(int64_t)bi * lds + bj] = s;

  const BlockDiv d = block_div(s);
  if (s == 0.0f) encode_block_rows<0, kStream>(v, d, full, q, N, K, ldq, row0, seg, col);
  else if (d.tiny) encode_block_rows<2, kStream>(v, d, full, q, N, K, ldq, row0, seg, col);
  else encode_block_rows<1, kStream>(v, d, full, q, N, K, ldq, row0, seg, col);
}

__global__ __launch_bounds__(256) void fp8_weight_block_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, int64_t ldw, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ scale, int64_t lds, int nbk) {
  const int bi = blockIdx.x / nbk;
  const int bj = blockIdx.x - bi * nbk;
  fp8_weight_block<false>(w, N, K, ldw, q, ldq, scale, lds, bi, bj);
}

// Several weights in one grid (a layer stack re-quantized after a training
// step): the jobs' blocks are numbered one after another, workgroup b takes
// block b; the job is found by a scan of the block prefix counts (uniform,
// at most kMaxWeightJobs entries, in the kernel arguments).  One launch
// instead of one per weight: small weights (a 10 MB k or v projection) no
// longer pay a launch ramp and drain of their own, and their blocks fill
// the machine beside the large ones.  A stack's codes outgrow the
// last-level cache, so they are stored non-temporal.
__global__ __launch_bounds__(256) void fp8_weight_block_multi_kernel(WeightJobs jobs) {
  const int b = blockIdx.x;
  int j = 0;
#pragma unroll 1
  while (j + 1 < jobs.count && b >= jobs.first[j + 1]) ++j;
  j = __builtin_amdgcn_readfirstlane(j);
  const int local = b - jobs.first[j];
  const int nbk = jobs.units_per_row[j];
  const int bi = local / nbk, bj = local - bi * nbk;
  const int64_t K = jobs.K[j];
  fp8_weight_block<true>(jobs.w[j], jobs.N[j], K, K, static_cast<uint8_t*>(jobs.q[j]), K,
                   jobs.scale[j], nbk, bi, bj);
}

// ---------------------------------------------------------------------------
// Activation groups.  16 lanes per (token, 128-feature group), each 16 lanes
// taking kActGroups consecutive groups (256 bytes apart in a row, or across
// a row end) whose loads are all issued before the first is used; a
// 256-thread workgroup covers 16 x kActGroups groups.  The amax never
// leaves the 16 lanes.  With one group per 16 lanes a workgroup holds only
// 4 KB in flight, and the 8192-token prefill activations streamed 10-17%
// slower than with four (four groups spaced a grid apart were slower
// still); but a decode batch, a few hundred workgroups at one group each,
// is latency bound, and four groups per 16 lanes lengthened it by ~1 us
// (4.2 -> 5.1 us at 64 x 3584).  So: one group while that grid has at most
// kActSmallGrid workgroups per CU, else four.
// ---------------------------------------------------------------------------
constexpr int kActGroups = 4;
constexpr int kActSmallGrid = 4;

template <bool kVec, int kGroups>
__global__ __launch_bounds__(256) void fp8_act_group_kernel(
    const uint16_t* __restrict__ a, int64_t M, int64_t K, uint8_t* __restrict__ q,
    float* __restrict__ scale, int64_t G) {
  const int tid = threadIdx.x;
  const int l16 = tid & 15;
  const int64_t gid0 = ((int64_t)blockIdx.x * 16 + (tid >> 4)) * kGroups;
  const int64_t total = M * G;
  if (gid0 >= total) return;       // whole 16-lane groups leave together
  uint4 v[kGroups];
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    const int64_t gid = gid0 + u;
    const int64_t mrow = gid / G;
    const int64_t col = (gid - mrow * G) * kBlock + l16 * 8;
    const uint16_t* src = a + mrow * K;
    if constexpr (kVec) {
      v[u] = (gid < total && col < K) ? load_once16(src + col) : make_uint4(0, 0, 0, 0);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (gid < total && col + e < K) ? (uint32_t)src[col + e] : 0u;
      v[u] = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                        h[6] | (h[7] << 16));
    }
  }
#pragma unroll
  for (int u = 0; u < kGroups; ++u) {
    const int64_t gid = gid0 + u;
    const int64_t mrow = gid / G;
    const int64_t col = (gid - mrow * G) * kBlock + l16 * 8;
    uint32_t m = 0;
    m = absmax_bf16x2(m, v[u].x);
    m = absmax_bf16x2(m, v[u].y);
    m = absmax_bf16x2(m, v[u].z);
    m = absmax_bf16x2(m, v[u].w);
    m = lane16_max_u32(absmax_fold(m));
    if (gid >= total) continue;
    const float s = div_rn(__uint_as_float(m << 16), kFp8Max);
    if (l16 == 0) scale[gid] = s;
    const uint2 c = e4m3_chunk_any(v[u], s, block_div(s));
    uint8_t* dst = q + mrow * K;
    if constexpr (kVec) {
      if (col < K) *reinterpret_cast<uint2*>(dst + col) = c;
    } else {
      const uint32_t cw[2] = {c.x, c.y};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (col + e < K) dst[col + e] = (uint8_t)(cw[e >> 2] >> (8 * (e & 3)));
    }
  }
}

hipError_t launch_fp8_weight_block_quant(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                         uint8_t* q, int64_t ldq, float* scale, int64_t lds,
                                         hipStream_t stream) {
  const int64_t nbn = (N + kBlock - 1) / kBlock, nbk = (K + kBlock - 1) / kBlock;
  const int64_t blocks = nbn * nbk;
  hipLaunchKernelGGL(fp8_weight_block_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w,
                     N, K, ldw, q, ldq, scale, lds, (int)nbk);
  return hipGetLastError();
}

hipError_t launch_fp8_weight_block_quant_multi(const WeightJobs& jobs, hipStream_t stream) {
  const int blocks = jobs.first[jobs.count];
  if (blocks > 0)
    hipLaunchKernelGGL(fp8_weight_block_multi_kernel, dim3((unsigned)blocks), dim3(256), 0,
                       stream, jobs);
  return hipGetLastError();
}

hipError_t launch_fp8_act_token_quant(const uint16_t* a, int64_t M, int64_t K, uint8_t* q,
                                      float* scale, hipStream_t stream) {
  const int64_t G = (K + kBlock - 1) / kBlock;
  const bool small = (M * G + 15) / 16 <= kActSmallGrid * (int64_t)compute_units();
  const int per = small ? 16 : 16 * kActGroups;
  const int64_t wgs = (M * G + per - 1) / per;
  const bool vec = K % 8 == 0;
  if (small && vec)
    hipLaunchKernelGGL((fp8_act_group_kernel<true, 1>), dim3((unsigned)wgs), dim3(256), 0, stream,
                       a, M, K, q, scale, G);
  else if (small)
    hipLaunchKernelGGL((fp8_act_group_kernel<false, 1>), dim3((unsigned)wgs), dim3(256), 0,
                       stream, a, M, K, q, scale, G);
  else if (vec)
    hipLaunchKernelGGL((fp8_act_group_kernel<true, kActGroups>), dim3((unsigned)wgs), dim3(256),
                       0, stream, a, M, K, q, scale, G);
  else
    hipLaunchKernelGGL((fp8_act_group_kernel<false, kActGroups>), dim3((unsigned)wgs),
                       dim3(256), 0, stream, a, M, K, q, scale, G);
  return hipGetLastError();
}

}  // namespace prr

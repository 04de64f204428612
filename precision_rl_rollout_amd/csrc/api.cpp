// The C ABI of libprr (declared in include/prr.h): argument checks, device
// checks, then one launcher call.  No allocation, no synchronization.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>
#include <cmath>

#include "launch.h"
#include "prr.h"

namespace {

constexpr int64_t kMaxDim = 0x7FFFFFFF;        // 2^31 - 1
constexpr int64_t kMaxInt8GemmK = 133143;      // 127^2 * K < 2^31
// Longest K of the dense GEMMs: the many-token kernel addresses one 256-row
// operand tile with 32-bit buffer offsets (256 K below 2^31 - 256), and it
// takes every shape the decode kernels decline.
constexpr int64_t kMaxGemmK = 8388480;         // 65535 * 128
constexpr int64_t kMaxGrid = 0x7FFFFFFF;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Dimensions: negative or too large -> INVALID_ARG.
prr_status check_dims(int64_t a, int64_t b, int64_t c = 0) {
  if (a < 0 || b < 0 || c < 0) return PRR_ERR_INVALID_ARG;
  if (a > kMaxDim || b > kMaxDim || c > kMaxDim) return PRR_ERR_INVALID_ARG;
  return PRR_OK;
}

// Pointers of a non-empty call: NULL -> INVALID_ARG, misaligned -> MISALIGNED.
prr_status check_ptrs(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if (p == nullptr) return PRR_ERR_INVALID_ARG;
  for (const void* p : ptrs)
    if (!aligned16(p)) return PRR_ERR_MISALIGNED;
  return PRR_OK;
}

// The current device must exist and be a gfx950.  The answer is cached per
// device ordinal (a HIP device's architecture does not change in a process).
prr_status check_device() {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return PRR_ERR_NO_DEVICE;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PRR_ERR_NO_DEVICE;
  static std::atomic<int> cache[64];   // 0 unknown, 1 gfx950, 2 other
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c != 0) return c == 1 ? PRR_OK : PRR_ERR_UNSUPPORTED_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return PRR_ERR_HIP;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) cache[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? PRR_OK : PRR_ERR_UNSUPPORTED_DEVICE;
}

prr_status from_hip(hipError_t e) { return e == hipSuccess ? PRR_OK : PRR_ERR_HIP; }

#define PRR_TRY(expr)                    \
  do {                                   \
    const prr_status st_ = (expr);       \
    if (st_ != PRR_OK) return st_;       \
  } while (0)

prr_status quant_common(const void* in, int64_t R, int64_t K, const void* out,
                        const void* scale, int64_t blocks) {
  PRR_TRY(check_dims(R, K));
  if (R == 0 || K == 0) return PRR_OK;
  PRR_TRY(check_ptrs({in, out, scale}));
  if (blocks > kMaxGrid) return PRR_ERR_UNSUPPORTED_SHAPE;
  return check_device();
}

}  // namespace

extern "C" {

prr_status fp8_weight_block_quant(const uint16_t* w_bf16, int64_t N, int64_t K, uint8_t* w_fp8,
                                  float* w_scale, hipStream_t stream) {
  if (N < 0 || K < 0) return PRR_ERR_INVALID_ARG;
  const int64_t blocks = ((N + 127) / 128) * ((K + 127) / 128);
  if (N == 0 || K == 0) return check_dims(N, K);
  PRR_TRY(quant_common(w_bf16, N, K, w_fp8, w_scale, blocks));
  return from_hip(prr::launch_fp8_weight_block_quant(w_bf16, N, K, K, w_fp8, K, w_scale,
                                                     (K + 127) / 128, stream));
}

prr_status fp8_weight_block_quant_into(const uint16_t* w_bf16, int64_t rows, int64_t cols,
                                       int64_t ld_w, uint8_t* q_fp8, int64_t ld_q, float* scale,
                                       int64_t ld_scale, hipStream_t stream) {
  if (rows < 0 || cols < 0) return PRR_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return check_dims(rows, cols);
  PRR_TRY(check_dims(rows, cols));
  PRR_TRY(check_dims(ld_w, ld_q, ld_scale));
  const int64_t nbk = (cols + 127) / 128;
  if (ld_w < cols || ld_q < cols || ld_scale < nbk) return PRR_ERR_INVALID_ARG;
  if (w_bf16 == nullptr || q_fp8 == nullptr || scale == nullptr) return PRR_ERR_INVALID_ARG;
  PRR_TRY(check_ptrs({w_bf16, q_fp8}));
  if (reinterpret_cast<uintptr_t>(scale) % 4 != 0) return PRR_ERR_MISALIGNED;
  if (((rows + 127) / 128) * nbk > kMaxGrid) return PRR_ERR_UNSUPPORTED_SHAPE;
  PRR_TRY(check_device());
  return from_hip(prr::launch_fp8_weight_block_quant(w_bf16, rows, cols, ld_w, q_fp8, ld_q,
                                                     scale, ld_scale, stream));
}

// Checks and work-unit layout shared by the two multi-weight calls.
static prr_status weight_jobs(const prr_weight_job* jobs, int64_t count, bool int8,
                              prr::WeightJobs* out) {
  if (count < 0 || count > PRR_MAX_WEIGHT_JOBS) return PRR_ERR_INVALID_ARG;
  if (count > 0 && jobs == nullptr) return PRR_ERR_INVALID_ARG;
  memset(out, 0, sizeof(*out));
  int64_t total = 0;
  for (int64_t i = 0; i < count; ++i) {
    const prr_weight_job& j = jobs[i];
    PRR_TRY(check_dims(j.N, j.K));
    if (j.N == 0 || (j.K == 0 && !int8)) continue;   // nothing to write
    if (j.K == 0) {
      PRR_TRY(check_ptrs({j.scale}));                 // INT8: zero scales only
    } else {
      PRR_TRY(check_ptrs({j.w_bf16, j.q, j.scale}));
    }
    const int c = out->count;
    out->w[c] = j.w_bf16;
    out->q[c] = j.q;
    out->scale[c] = j.scale;
    out->N[c] = j.N;
    out->K[c] = j.K;
    int64_t units;
    if (int8) {
      const int cls = prr::int8_row_class(j.K);
      const int per = prr::int8_rows_per_unit(cls);
      out->units_per_row[c] = cls;
      units = (j.N + per - 1) / per;
    } else {
      const int64_t nbk = (j.K + 127) / 128;
      out->units_per_row[c] = (int)nbk;
      units = ((j.N + 127) / 128) * nbk;
    }
    out->first[c] = (int)total;
    total += units;
    if (total > kMaxGrid) return PRR_ERR_UNSUPPORTED_SHAPE;
    out->count = c + 1;
  }
  out->first[out->count] = (int)total;
  // The scan in the kernels reads first[count]; unused slots stay zero.
  return PRR_OK;
}

prr_status fp8_weight_block_quant_multi(const prr_weight_job* jobs, int64_t count,
                                        hipStream_t stream) {
  prr::WeightJobs wj;
  PRR_TRY(weight_jobs(jobs, count, false, &wj));
  if (wj.first[wj.count] == 0) return PRR_OK;
  PRR_TRY(check_device());
  return from_hip(prr::launch_fp8_weight_block_quant_multi(wj, stream));
}

prr_status int8_weight_channel_quant_multi(const prr_weight_job* jobs, int64_t count,
                                           hipStream_t stream) {
  prr::WeightJobs wj;
  PRR_TRY(weight_jobs(jobs, count, true, &wj));
  if (wj.first[wj.count] == 0) return PRR_OK;
  PRR_TRY(check_device());
  return from_hip(prr::launch_int8_weight_channel_quant_multi(wj, stream));
}

prr_status fp8_act_token_quant(const uint16_t* a_bf16, int64_t M, int64_t K, uint8_t* a_fp8,
                               float* a_scale, hipStream_t stream) {
  if (M < 0 || K < 0) return PRR_ERR_INVALID_ARG;
  if (M == 0 || K == 0) return check_dims(M, K);
  const int64_t wgs = (M * ((K + 127) / 128) + 15) / 16;
  PRR_TRY(quant_common(a_bf16, M, K, a_fp8, a_scale, wgs));
  return from_hip(prr::launch_fp8_act_token_quant(a_bf16, M, K, a_fp8, a_scale, stream));
}

prr_status int8_weight_channel_quant(const uint16_t* w_bf16, int64_t N, int64_t K, int8_t* w_i8,
                                     float* w_scale, hipStream_t stream) {
  if (N < 0 || K < 0) return PRR_ERR_INVALID_ARG;
  if (N == 0 || K == 0) {
    // K == 0 with N > 0: every row is empty, amax = 0, scale = 0.
    PRR_TRY(check_dims(N, K));
    if (N == 0) return PRR_OK;
    PRR_TRY(check_ptrs({w_scale}));
    PRR_TRY(check_device());
    // The row kernel with K == 0 writes scale 0 and reads no element.
    return from_hip(prr::launch_int8_weight_channel_quant(w_bf16, N, 0, w_i8, w_scale, stream));
  }
  PRR_TRY(quant_common(w_bf16, N, K, w_i8, w_scale, N));
  return from_hip(prr::launch_int8_weight_channel_quant(w_bf16, N, K, w_i8, w_scale, stream));
}

prr_status int8_act_token_quant(const uint16_t* a_bf16, int64_t M, int64_t K, int8_t* a_i8,
                                float* a_scale, hipStream_t stream) {
  if (M < 0 || K < 0) return PRR_ERR_INVALID_ARG;
  if (M == 0 || K == 0) {
    PRR_TRY(check_dims(M, K));
    if (M == 0) return PRR_OK;
    PRR_TRY(check_ptrs({a_scale}));
    PRR_TRY(check_device());
    return from_hip(prr::launch_int8_act_token_quant(a_bf16, M, 0, a_i8, a_scale, stream));
  }
  PRR_TRY(quant_common(a_bf16, M, K, a_i8, a_scale, M));
  return from_hip(prr::launch_int8_act_token_quant(a_bf16, M, K, a_i8, a_scale, stream));
}

static prr_status gemm_common(const void* a, const void* sa, const void* w, const void* sw,
                              int64_t M, int64_t N, int64_t K, const void* c, bool int8) {
  PRR_TRY(check_dims(M, N, K));
  if (K % 128 != 0 || K > kMaxGemmK) return PRR_ERR_UNSUPPORTED_SHAPE;
  if (int8 && K > kMaxInt8GemmK) return PRR_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0) return PRR_OK;
  if (K == 0) {
    PRR_TRY(check_ptrs({c}));
    if ((M * N + 255) / 256 > kMaxGrid) return PRR_ERR_UNSUPPORTED_SHAPE;
  } else {
    PRR_TRY(check_ptrs({a, sa, w, sw, c}));
    if ((N + 15) / 16 > kMaxGrid || ((N + 127) / 128) * ((M + 127) / 128) > kMaxGrid)
      return PRR_ERR_UNSUPPORTED_SHAPE;
  }
  return check_device();
}

prr_status w8a8_block_gemm(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                           const float* w_scale, int64_t M, int64_t N, int64_t K,
                           uint16_t* c_bf16, hipStream_t stream) {
  PRR_TRY(gemm_common(a_fp8, a_scale, w_fp8, w_scale, M, N, K, c_bf16, false));
  if (M == 0 || N == 0) return PRR_OK;
  return from_hip(
      prr::launch_w8a8_block_gemm(a_fp8, a_scale, w_fp8, w_scale, M, N, K, c_bf16, stream));
}

prr_status w8a8_int8_channel_gemm(const int8_t* a_i8, const float* a_scale, const int8_t* w_i8,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K,
                                  uint16_t* c_bf16, hipStream_t stream) {
  PRR_TRY(gemm_common(a_i8, a_scale, w_i8, w_scale, M, N, K, c_bf16, true));
  if (M == 0 || N == 0) return PRR_OK;
  return from_hip(
      prr::launch_w8a8_int8_channel_gemm(a_i8, a_scale, w_i8, w_scale, M, N, K, c_bf16, stream));
}

prr_status w8a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t* bytes) {
  if (bytes == nullptr) return PRR_ERR_INVALID_ARG;
  *bytes = 0;
  PRR_TRY(check_dims(M, N, K));
  if (K % 128 != 0) return PRR_ERR_UNSUPPORTED_SHAPE;
  if (M == 0 || N == 0 || K == 0) return PRR_OK;
  PRR_TRY(check_device());
  prr::SplitPlan plan;
  prr::PrefillTailPlan tail;
  if (prr::splitk_plan(M, N, K, &plan)) *bytes = plan.bytes;
  else if (prr::prefill_tail_plan(M, N, K, &tail)) *bytes = tail.bytes;
  return PRR_OK;
}

prr_status w8a8_block_gemm_ws(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                              const float* w_scale, int64_t M, int64_t N, int64_t K,
                              uint16_t* c_bf16, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream) {
  if (workspace_bytes < 0) return PRR_ERR_INVALID_ARG;
  if (workspace != nullptr && workspace_bytes > 0 && M > 0 && N > 0)
    PRR_TRY(check_ptrs({workspace}));
  PRR_TRY(gemm_common(a_fp8, a_scale, w_fp8, w_scale, M, N, K, c_bf16, false));
  if (M == 0 || N == 0) return PRR_OK;
  hipError_t err = hipSuccess;
  if (K > 0 && prr::launch_gemm_decode_splitk<false>(a_fp8, a_scale, w_fp8, w_scale, M, N, K,
                                                      static_cast<float*>(workspace),
                                                      workspace_bytes, c_bf16, stream, &err))
    return from_hip(err);
  if (K > 0 && prr::launch_gemm_prefill_ws<false>(a_fp8, a_scale, w_fp8, w_scale, M, N, K, c_bf16,
                                                   static_cast<float*>(workspace),
                                                   workspace_bytes, stream, &err))
    return from_hip(err);
  return from_hip(
      prr::launch_w8a8_block_gemm(a_fp8, a_scale, w_fp8, w_scale, M, N, K, c_bf16, stream));
}

prr_status w8a8_block_gemm_scratch(const uint8_t* a_fp8, const float* a_scale,
                                   const uint8_t* w_fp8, const float* w_scale, int64_t M,
                                   int64_t N, int64_t K, uint16_t* c_bf16, hipStream_t stream) {
  PRR_TRY(gemm_common(a_fp8, a_scale, w_fp8, w_scale, M, N, K, c_bf16, false));
  if (M == 0 || N == 0) return PRR_OK;
  prr::SplitPlan plan;
  if (K > 0 && prr::splitk_plan(M, N, K, &plan)) {
    if (plan.bytes > prr::kScratchBytes) return PRR_ERR_UNSUPPORTED_SHAPE;
    hipError_t err = hipSuccess;
    float* ws = prr::scratch_ptr(&err);
    if (ws == nullptr) return PRR_ERR_HIP;
    if (prr::launch_gemm_decode_splitk<false>(a_fp8, a_scale, w_fp8, w_scale, M, N, K, ws,
                                              prr::kScratchBytes, c_bf16, stream, &err))
      return from_hip(err);
  }
  // No split for this shape: the one-pass kernels, which use no scratch.
  return from_hip(
      prr::launch_w8a8_block_gemm(a_fp8, a_scale, w_fp8, w_scale, M, N, K, c_bf16, stream));
}

prr_status w8a8_int8_channel_gemm_ws(const int8_t* a_i8, const float* a_scale,
                                     const int8_t* w_i8, const float* w_scale, int64_t M,
                                     int64_t N, int64_t K, uint16_t* c_bf16, void* workspace,
                                     int64_t workspace_bytes, hipStream_t stream) {
  if (workspace_bytes < 0) return PRR_ERR_INVALID_ARG;
  if (workspace != nullptr && workspace_bytes > 0 && M > 0 && N > 0)
    PRR_TRY(check_ptrs({workspace}));
  PRR_TRY(gemm_common(a_i8, a_scale, w_i8, w_scale, M, N, K, c_bf16, true));
  if (M == 0 || N == 0) return PRR_OK;
  hipError_t err = hipSuccess;
  if (K > 0 && prr::launch_gemm_decode_splitk<true>(
                   reinterpret_cast<const uint8_t*>(a_i8), a_scale,
                   reinterpret_cast<const uint8_t*>(w_i8), w_scale, M, N, K,
                   static_cast<float*>(workspace), workspace_bytes, c_bf16, stream, &err))
    return from_hip(err);
  if (K > 0 && prr::launch_gemm_prefill_ws<true>(
                   reinterpret_cast<const uint8_t*>(a_i8), a_scale,
                   reinterpret_cast<const uint8_t*>(w_i8), w_scale, M, N, K, c_bf16,
                   static_cast<float*>(workspace), workspace_bytes, stream, &err))
    return from_hip(err);
  return from_hip(
      prr::launch_w8a8_int8_channel_gemm(a_i8, a_scale, w_i8, w_scale, M, N, K, c_bf16, stream));
}

prr_status w8a8_block_gemm_grouped(const uint8_t* a_fp8, const float* a_scale,
                                   const uint8_t* w_fp8, const float* w_scale,
                                   const int64_t* expert_offsets, int64_t E, int64_t M, int64_t N,
                                   int64_t K, int64_t max_rows_per_expert, uint16_t* c_bf16,
                                   hipStream_t stream) {
  PRR_TRY(check_dims(E, M, N));
  PRR_TRY(check_dims(K, max_rows_per_expert));
  if (K % 128 != 0 || K == 0) return PRR_ERR_UNSUPPORTED_SHAPE;
  if (E == 0 || M == 0 || N == 0) return PRR_OK;
  PRR_TRY(check_ptrs({a_fp8, a_scale, w_fp8, w_scale, expert_offsets, c_bf16}));
  PRR_TRY(check_device());
  hipError_t err = hipSuccess;
  if (!prr::launch_gemm_grouped(a_fp8, a_scale, w_fp8, w_scale, expert_offsets, E, M, N, K,
                                max_rows_per_expert, c_bf16, stream, &err))
    return PRR_ERR_UNSUPPORTED_SHAPE;
  return from_hip(err);
}

prr_status fp8_kv_scale_recalibrate(const uint16_t* x_bf16, int64_t T, int64_t C, float* scale,
                                    hipStream_t stream) {
  PRR_TRY(check_dims(T, C));
  const int64_t n = T * C;
  if (n > 0) {
    PRR_TRY(check_ptrs({x_bf16, scale}));
  } else {
    PRR_TRY(check_ptrs({scale}));
  }
  PRR_TRY(check_device());
  return from_hip(prr::launch_fp8_kv_scale_recalibrate(x_bf16, n, scale, stream));
}

prr_status fp8_kv_cache_write(const uint16_t* kv_bf16, const int64_t* slot_mapping, int64_t T,
                              int64_t C, const float* scale, uint8_t* cache, int64_t num_slots,
                              hipStream_t stream) {
  PRR_TRY(check_dims(T, C, num_slots));
  if (T == 0 || C == 0 || num_slots == 0) return PRR_OK;
  PRR_TRY(check_ptrs({kv_bf16, slot_mapping, scale, cache}));
  PRR_TRY(check_device());
  return from_hip(
      prr::launch_fp8_kv_cache_write(kv_bf16, slot_mapping, T, C, scale, cache, num_slots, stream));
}

// Checks of the write + recalibration calls; fills *kj.  Per job: new_scale
// always (an empty batch still writes 0); the rows, scale and workspace
// when T x C > 0, the cache when num_slots > 0; new_scale words distinct.
static prr_status kv_recal_jobs(const prr_kv_job* jobs, int64_t count,
                                const int64_t* slot_mapping, int64_t T, int64_t C,
                                int64_t num_slots, const void* workspace, int64_t workspace_bytes,
                                prr::KvJobs* kj) {
  static_assert(PRR_KV_RECAL_WORKSPACE_BYTES == 4 * prr::kKvRecalParts, "partials workspace");
  static_assert(PRR_MAX_KV_JOBS == prr::kMaxKvJobs, "job limit");
  PRR_TRY(check_dims(T, C, num_slots));
  if (count < 0 || count > PRR_MAX_KV_JOBS || workspace_bytes < 0) return PRR_ERR_INVALID_ARG;
  if (count > 0 && jobs == nullptr) return PRR_ERR_INVALID_ARG;
  const bool rows = T > 0 && C > 0;
  if (rows && count > 0) {
    PRR_TRY(check_ptrs({slot_mapping, workspace}));
    if (workspace_bytes < count * (int64_t)PRR_KV_RECAL_WORKSPACE_BYTES) return PRR_ERR_INVALID_ARG;
  }
  kj->count = (int)count;
  for (int64_t j = 0; j < count; ++j) {
    const prr_kv_job& jb = jobs[j];
    PRR_TRY(check_ptrs({jb.new_scale}));
    if (rows) {
      PRR_TRY(check_ptrs({jb.kv_bf16, jb.scale}));
      if (num_slots > 0) PRR_TRY(check_ptrs({jb.cache}));
    }
    for (int64_t i = 0; i < j; ++i)
      if (jobs[i].new_scale == jb.new_scale) return PRR_ERR_INVALID_ARG;
    kj->kv[j] = jb.kv_bf16;
    kj->scale[j] = jb.scale;
    kj->cache[j] = num_slots > 0 ? jb.cache : nullptr;
    kj->new_scale[j] = jb.new_scale;
  }
  return PRR_OK;
}

prr_status fp8_kv_cache_write_recalibrate(const uint16_t* kv_bf16,
                                          const int64_t* slot_mapping, int64_t T, int64_t C,
                                          const float* scale, uint8_t* cache, int64_t num_slots,
                                          float* new_scale, void* workspace,
                                          int64_t workspace_bytes, hipStream_t stream) {
  const prr_kv_job job{kv_bf16, scale, cache, new_scale};
  prr::KvJobs kj;
  PRR_TRY(kv_recal_jobs(&job, 1, slot_mapping, T, C, num_slots, workspace, workspace_bytes, &kj));
  PRR_TRY(check_device());
  return from_hip(prr::launch_fp8_kv_cache_write_recalibrate(
      kj, slot_mapping, T, C, num_slots, static_cast<uint32_t*>(workspace), stream));
}

prr_status fp8_kv_cache_write_recalibrate_multi(const prr_kv_job* jobs, int64_t count,
                                                const int64_t* slot_mapping, int64_t T,
                                                int64_t C, int64_t num_slots, void* workspace,
                                                int64_t workspace_bytes, hipStream_t stream) {
  prr::KvJobs kj;
  PRR_TRY(kv_recal_jobs(jobs, count, slot_mapping, T, C, num_slots, workspace, workspace_bytes,
                        &kj));
  if (count == 0) return PRR_OK;
  PRR_TRY(check_device());
  return from_hip(prr::launch_fp8_kv_cache_write_recalibrate(
      kj, slot_mapping, T, C, num_slots, static_cast<uint32_t*>(workspace), stream));
}

prr_status tis_token_weights(const float* logp_train, const float* logp_rollout,
                             const uint8_t* mask, int64_t B, int64_t T, float cap, int mode,
                             float* weights, float* row_stats, double* totals,
                             hipStream_t stream) {
  PRR_TRY(check_dims(B, T));
  if (!(cap > 0.0f) || (mode != PRR_IS_TRUNCATE && mode != PRR_IS_MASK)) return PRR_ERR_INVALID_ARG;
  if (totals != nullptr && row_stats == nullptr && B > 0) return PRR_ERR_INVALID_ARG;
  if (T > (int64_t(1) << 24)) return PRR_ERR_UNSUPPORTED_SHAPE;   // counts kept exact in fp32
  if (B > 0 && T > 0) PRR_TRY(check_ptrs({logp_train, logp_rollout, mask, weights}));
  if (B > 0 && row_stats != nullptr) PRR_TRY(check_ptrs({row_stats}));
  if (totals != nullptr) PRR_TRY(check_ptrs({totals}));
  if (B == 0 && totals == nullptr) return PRR_OK;
  if (T == 0 && row_stats == nullptr && totals == nullptr) return PRR_OK;
  PRR_TRY(check_device());
  // fl32(ln C), from the fp64 logarithm rounded once; +inf for C = +inf.
  const float lncap = std::isinf(cap) ? cap : (float)std::log((double)cap);
  return from_hip(prr::launch_tis_token_weights(logp_train, logp_rollout, mask, B, T, cap, lncap,
                                                mode, weights, row_stats, totals, stream));
}

// Checks shared by the two attention calls; PRR_OK with *empty set when
// there is nothing to compute.
static prr_status attention_common(const uint16_t* q_bf16, const float* q_scale,
                                   const uint8_t* k_cache, const uint8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, const int32_t* seq_lens, int64_t B,
                                   int64_t Hq, int64_t Hkv, int64_t D, int64_t page,
                                   int64_t max_blocks, int64_t num_slots, float softmax_scale,
                                   uint16_t* out_bf16, bool* empty) {
  *empty = false;
  PRR_TRY(check_dims(B, Hq, Hkv));
  PRR_TRY(check_dims(D, page, max_blocks));
  PRR_TRY(check_dims(num_slots, 0));
  if (!std::isfinite(softmax_scale)) return PRR_ERR_INVALID_ARG;
  if (B == 0 || Hq == 0) {
    *empty = true;
    return PRR_OK;
  }
  if (Hkv == 0 || page == 0 || max_blocks == 0) return PRR_ERR_INVALID_ARG;
  if (D != 128 || Hq % Hkv != 0 || Hq / Hkv > 8) return PRR_ERR_UNSUPPORTED_SHAPE;
  if (B * Hkv > kMaxGrid || page > (int64_t(1) << 20) || max_blocks * page > (int64_t(1) << 40))
    return PRR_ERR_UNSUPPORTED_SHAPE;
  PRR_TRY(check_ptrs({q_bf16, q_scale, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens,
                      out_bf16}));
  return check_device();
}

prr_status fp8_kv_decode_attention(const uint16_t* q_bf16, const float* q_scale,
                                   const uint8_t* k_cache, const uint8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page,
                                   int64_t max_blocks, int64_t num_slots, float softmax_scale,
                                   uint16_t* out_bf16, hipStream_t stream) {
  bool empty = false;
  PRR_TRY(attention_common(q_bf16, q_scale, k_cache, v_cache, k_scale, v_scale, block_table,
                           seq_lens, B, Hq, Hkv, D, page, max_blocks, num_slots, softmax_scale,
                           out_bf16, &empty));
  if (empty) return PRR_OK;
  return from_hip(prr::launch_fp8_decode_attention(q_bf16, q_scale, k_cache, v_cache, k_scale,
                                                   v_scale, block_table, seq_lens, B, Hq, Hkv,
                                                   page, max_blocks, num_slots, softmax_scale,
                                                   out_bf16, stream));
}

prr_status fp8_kv_decode_attention_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                                  int64_t* bytes) {
  if (bytes == nullptr) return PRR_ERR_INVALID_ARG;
  *bytes = 0;
  PRR_TRY(check_dims(B, Hq, Hkv));
  PRR_TRY(check_dims(D, 0, 0));
  if (B == 0 || Hq == 0) return PRR_OK;
  PRR_TRY(check_device());
  *bytes = prr::fp8_decode_attention_workspace_bytes(B, Hq, Hkv, D);
  return PRR_OK;
}

prr_status fp8_kv_decode_attention_ws(const uint16_t* q_bf16, const float* q_scale,
                                      const uint8_t* k_cache, const uint8_t* v_cache,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page,
                                      int64_t max_blocks, int64_t num_slots, float softmax_scale,
                                      uint16_t* out_bf16, void* workspace,
                                      int64_t workspace_bytes, hipStream_t stream) {
  if (workspace_bytes < 0) return PRR_ERR_INVALID_ARG;
  if (workspace != nullptr && workspace_bytes > 0 && B > 0 && Hq > 0)
    PRR_TRY(check_ptrs({workspace}));
  bool empty = false;
  PRR_TRY(attention_common(q_bf16, q_scale, k_cache, v_cache, k_scale, v_scale, block_table,
                           seq_lens, B, Hq, Hkv, D, page, max_blocks, num_slots, softmax_scale,
                           out_bf16, &empty));
  if (empty) return PRR_OK;
  hipError_t err = hipSuccess;
  if (prr::launch_fp8_decode_attention_span(q_bf16, q_scale, k_cache, v_cache, k_scale, v_scale,
                                            block_table, seq_lens, B, Hq, Hkv, page, max_blocks,
                                            num_slots, softmax_scale, out_bf16, workspace,
                                            workspace_bytes, stream, &err))
    return from_hip(err);
  return from_hip(prr::launch_fp8_decode_attention(q_bf16, q_scale, k_cache, v_cache, k_scale,
                                                   v_scale, block_table, seq_lens, B, Hq, Hkv,
                                                   page, max_blocks, num_slots, softmax_scale,
                                                   out_bf16, stream));
}

const char* prr_status_string(prr_status status) {
  switch (status) {
    case PRR_OK: return "PRR_OK";
    case PRR_ERR_INVALID_ARG: return "PRR_ERR_INVALID_ARG";
    case PRR_ERR_UNSUPPORTED_SHAPE: return "PRR_ERR_UNSUPPORTED_SHAPE";
    case PRR_ERR_MISALIGNED: return "PRR_ERR_MISALIGNED";
    case PRR_ERR_NO_DEVICE: return "PRR_ERR_NO_DEVICE";
    case PRR_ERR_UNSUPPORTED_DEVICE: return "PRR_ERR_UNSUPPORTED_DEVICE";
    case PRR_ERR_HIP: return "PRR_ERR_HIP";
  }
  return "PRR_ERR_UNKNOWN";
}

int prr_abi_version(void) { return PRR_ABI_VERSION; }

}  // extern "C"

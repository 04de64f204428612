// Kernel launchers of libprr, called by the C ABI after argument checks.
// Each enqueues its kernels on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prr {

// (row strides: ldw input elements, ldq code bytes, lds scale floats)
hipError_t launch_fp8_weight_block_quant(const uint16_t* w, int64_t N, int64_t K, int64_t ldw,
                                         uint8_t* q, int64_t ldq, float* scale, int64_t lds,
                                         hipStream_t stream);
hipError_t launch_fp8_act_token_quant(const uint16_t* a, int64_t M, int64_t K, uint8_t* q,
                                      float* scale, hipStream_t stream);

// Several whole weights Wt [N, K] quantized in one launch (passed by value
// in the kernel arguments).  first[j] is the first work unit of job j
// (first[count] = total): FP8, 128 x 128 blocks (units_per_row = blocks
// per block row); INT8, row groups of a class chosen per job.
constexpr int kMaxWeightJobs = 16;
struct WeightJobs {
  const uint16_t* w[kMaxWeightJobs];
  void* q[kMaxWeightJobs];
  float* scale[kMaxWeightJobs];
  int64_t N[kMaxWeightJobs];
  int64_t K[kMaxWeightJobs];
  int units_per_row[kMaxWeightJobs];   // FP8: blocks per block row; INT8: row class
  int first[kMaxWeightJobs + 1];
  int count;
};
hipError_t launch_fp8_weight_block_quant_multi(const WeightJobs& jobs, hipStream_t stream);
hipError_t launch_int8_weight_channel_quant_multi(const WeightJobs& jobs, hipStream_t stream);
// INT8 row class of a weight with K columns and the rows one work unit takes.
int int8_row_class(int64_t K);
int int8_rows_per_unit(int cls);
hipError_t launch_w8a8_block_gemm(const uint8_t* A, const float* sa, const uint8_t* W,
                                  const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* C,
                                  hipStream_t stream);
hipError_t launch_int8_weight_channel_quant(const uint16_t* w, int64_t N, int64_t K, int8_t* q,
                                            float* scale, hipStream_t stream);
hipError_t launch_int8_act_token_quant(const uint16_t* a, int64_t M, int64_t K, int8_t* q,
                                       float* scale, hipStream_t stream);
hipError_t launch_w8a8_int8_channel_gemm(const int8_t* A, const float* sa, const int8_t* W,
                                         const float* sw, int64_t M, int64_t N, int64_t K,
                                         uint16_t* C, hipStream_t stream);

// FP8 KV cache: recalibration over n = T x C values (the scale word doubles
// as the reduction's accumulator) and quantize-on-write.
hipError_t launch_fp8_kv_scale_recalibrate(const uint16_t* x, int64_t n, float* scale,
                                           hipStream_t stream);
hipError_t launch_fp8_kv_cache_write(const uint16_t* kv, const int64_t* slots, int64_t T,
                                     int64_t C, const float* scale, uint8_t* cache,
                                     int64_t num_slots, hipStream_t stream);
// Both in one pass over the rows, for up to kMaxKvJobs tensors sharing the
// slot mapping (K and V of a step): job j's rows written into cache[j] with
// scale[j], and new_scale[j] recalibrated from them through per-workgroup
// maxima in part + j kKvRecalParts (at most kKvRecalParts words each,
// written before they are read).
constexpr int kKvRecalParts = 2048;
constexpr int kMaxKvJobs = 16;
struct KvJobs {
  const uint16_t* kv[kMaxKvJobs];
  const float* scale[kMaxKvJobs];
  uint8_t* cache[kMaxKvJobs];
  float* new_scale[kMaxKvJobs];
  int count;
};
hipError_t launch_fp8_kv_cache_write_recalibrate(const KvJobs& jobs, const int64_t* slots,
                                                 int64_t T, int64_t C, int64_t num_slots,
                                                 uint32_t* part, hipStream_t stream);

hipError_t launch_tis_token_weights(const float* lp_train, const float* lp_rollout,
                                    const uint8_t* mask, int64_t B, int64_t T, float cap,
                                    float lncap, int mode, float* w, float* row_stats,
                                    double* totals, hipStream_t stream);

hipError_t launch_fp8_decode_attention(const uint16_t* q, const float* q_scale,
                                       const uint8_t* k_cache, const uint8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       int64_t B, int64_t Hq, int64_t Hkv, int64_t page,
                                       int64_t max_blocks, int64_t num_slots,
                                       float softmax_scale, uint16_t* out, hipStream_t stream);

// Decode attention split over the batch's tokens with a caller workspace:
// the bytes it needs (0: this shape takes the one-pass kernel), and the
// launch (false, nothing launched, when the shape has no split or the
// workspace is missing or too small).
int64_t fp8_decode_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D);
bool launch_fp8_decode_attention_span(const uint16_t* q, const float* q_scale,
                                      const uint8_t* k_cache, const uint8_t* v_cache,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int64_t B, int64_t Hq, int64_t Hkv, int64_t page,
                                      int64_t max_blocks, int64_t num_slots, float softmax_scale,
                                      uint16_t* out, void* ws, int64_t ws_bytes,
                                      hipStream_t stream, hipError_t* err);

// Split-K decode GEMM plan: S K-slices, G workgroups, MT m-tiles, pw K
// blocks per wave, `bytes` of fp32 workspace.  False: no split for this
// shape (the one-pass kernels handle it).
struct SplitPlan {
  int S, G, MT, pw;
  int64_t bytes;
};
bool splitk_plan(int64_t M, int64_t N, int64_t K, SplitPlan* plan);

// Split-K decode GEMM into the caller's workspace; false if the shape has no
// split plan or the workspace is missing or too small (nothing launched).
template <bool kInt8>
bool launch_gemm_decode_splitk(const uint8_t* A, const float* sa, const uint8_t* W,
                               const float* sw, int64_t M, int64_t N, int64_t K, float* ws,
                               int64_t ws_bytes, uint16_t* C, hipStream_t stream,
                               hipError_t* err);

// Compute units of the current device (cached per device; 256 if unknown).
int compute_units();

// The library's static scratch array (a file-scope __device__ array, one per
// device the library runs on, held until the process ends): its size, and
// its device address on the current device, looked up once per device with
// hipGetSymbolAddress (nullptr, with *err set, if that fails).  Used by the
// allocation-free split-K GEMM entry point only.
constexpr int64_t kScratchBytes = int64_t(16) << 20;
float* scratch_ptr(hipError_t* err);

// Decode-sized W8A8 GEMM (activation-resident, persistent).  Returns false,
// launching nothing, when the shape is outside what it handles.
template <bool kInt8>
bool launch_gemm_decode(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                        int64_t M, int64_t N, int64_t K, uint16_t* C, hipStream_t stream,
                        hipError_t* err);

// Grouped (mixture-of-experts) FP8 GEMM on the decode machinery; rows_hint
// bounds the rows per expert for the register tiling (larger groups run in
// 64-row chunks).  Returns false, launching nothing, when K is too large.
bool launch_gemm_grouped(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                         const int64_t* offsets, int64_t E, int64_t M, int64_t N, int64_t K,
                         int64_t rows_hint, uint16_t* C, hipStream_t stream, hipError_t* err);

// Many-token W8A8 GEMM (256 x 256 tiles, LDS ring fed by direct-to-LDS
// loads).  Returns false, launching nothing, outside the shapes it handles.
template <bool kInt8>
bool launch_gemm_prefill(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                         int64_t M, int64_t N, int64_t K, uint16_t* C, hipStream_t stream,
                         hipError_t* err);

// With a caller workspace, more than 128 rows: the many-token kernel with
// the last partial round's tile columns split over K (fp32 partial sums in
// the workspace, added by a second kernel).  The plan: columns [0, n_split)
// in whole rounds of 256-wide tiles, the rest in S slices; bytes of
// workspace.  Returns false (launching nothing) when the shape has no such
// round, its K is short, or the workspace is missing or too small.
struct PrefillTailPlan {
  int64_t n_split;
  int S;
  int64_t bytes;
};
bool prefill_tail_plan(int64_t M, int64_t N, int64_t K, PrefillTailPlan* plan);
template <bool kInt8>
bool launch_gemm_prefill_ws(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                            int64_t M, int64_t N, int64_t K, uint16_t* C, float* ws,
                            int64_t ws_bytes, hipStream_t stream, hipError_t* err);

}  // namespace prr

// Kernel launchers of libprr, called by the C ABI after argument checks.
// Each enqueues its kernels on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace prr {

hipError_t launch_fp8_weight_block_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* q,
                                         float* scale, hipStream_t stream);
hipError_t launch_fp8_act_token_quant(const uint16_t* a, int64_t M, int64_t K, uint8_t* q,
                                      float* scale, hipStream_t stream);
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

// Compute units of the current device (cached per device; 256 if unknown).
int compute_units();

// Decode-sized W8A8 GEMM (activation-resident, persistent).  Returns false,
// launching nothing, when the shape is outside what it handles.
template <bool kInt8>
bool launch_gemm_decode(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                        int64_t M, int64_t N, int64_t K, uint16_t* C, hipStream_t stream,
                        hipError_t* err);

// Many-token W8A8 GEMM (256 x 256 tiles, LDS ring fed by direct-to-LDS
// loads).  Returns false, launching nothing, outside the shapes it handles.
template <bool kInt8>
bool launch_gemm_prefill(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                         int64_t M, int64_t N, int64_t K, uint16_t* C, hipStream_t stream,
                         hipError_t* err);

}  // namespace prr

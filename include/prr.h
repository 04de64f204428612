/*
 * prr.h -- C ABI of libprr.so: MI355X (gfx950) kernels for 8-bit rollout.
 *
 * The calls implement the per-step re-quantization of freshly updated bf16
 * policy weights and activations into FP8 e4m3 with block scales (whole
 * weights, or shards quantized into place as a weight synchronization
 * delivers them), the W8A8 block-scaled linear layer with bf16 output (also
 * grouped over the experts of a mixture-of-experts layer), an INT8
 * per-channel variant of both, the FP8 KV cache (per-step scale
 * recalibration, quantize-on-write, decode attention over the paged
 * cache), and token-level TIS / MIS importance weights.  Sources:
 *   - "FP8-RL: A Practical and Stable Low-Precision Stack for LLM
 *     Reinforcement Learning", abstract: policy weights change every step
 *     and must be quantized again every step; item (i): FP8 W8A8
 *     linear-layer rollout with blockwise FP8 quantization; item (ii): FP8
 *     KV cache with per-step QKV scale recalibration; item (iii):
 *     token-level TIS / MIS rollout correction.
 *   - FlashRL article ("FlashRL: 8Bit Rollouts, Full Power RL"), sections
 *     on rollout quantization and online quantization with parameter
 *     updates: INT8 and FP8 rollout.
 * Block sizes (128 x 128 weight blocks, 1 x 128 activation groups), the
 * e4m3 format with scale amax / 448, the INT8 per-channel granularity and
 * the per-tensor KV-cache scale are fixed by this library; the pages do not
 * state them.
 *
 * Conventions shared by every call
 * --------------------------------
 * Data:
 *   - bf16 tensors are raw uint16_t bit patterns; FP8 tensors are OCP e4m3
 *     codes (uint8_t: 1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
 *     largest finite 448, 0x7F/0xFF NaN -- never produced); INT8 codes are
 *     int8_t in [-127, 127]; scales are IEEE binary32.
 *   - Every matrix is dense row-major.  Weights are stored as Wt [N, K]
 *     (output channel x input feature, K contiguous) -- the transpose of the
 *     logical W [K, N] of C = A W.  128 x 128 blocks are square, so the
 *     blocking of Wt is the blocking of W.
 *   - Quantized values follow one definition, bit for bit:
 *       FP8:  s = fl32(amax / 448), q = E4M3_saturating_RNE(fl32(x / s));
 *       INT8: s = fl32(amax / 127), q = clamp(RNE(fl32(x / s)), -127, 127);
 *     fl32 is an IEEE binary32 operation, correctly rounded, subnormals
 *     kept.  An all-zero block/row has s = 0: FP8 codes are the inputs'
 *     signed zeros (0x00 / 0x80), INT8 codes are 0.  Partial edge blocks
 *     take amax over their valid elements.
 *   - Inputs must be finite; non-finite inputs give unspecified (but
 *     memory-safe) results.
 * Pointers and memory:
 *   - Every pointer is a device pointer on the current HIP device, 16-byte
 *     aligned (PRR_ERR_MISALIGNED otherwise; fp8_weight_block_quant_into's
 *     scale pointer needs 4 bytes).  The caller allocates and owns
 *     every buffer; the library allocates nothing, frees nothing and keeps
 *     no pointer after the call returns.  Inputs and outputs must not
 *     overlap.
 *   - A call whose output is empty (a zero dimension) returns PRR_OK and
 *     touches no memory; its pointers may then be NULL.
 * Execution:
 *   - Every call only enqueues work on `stream` (NULL = the null stream)
 *     and returns without synchronizing.  Buffers must stay valid until
 *     that work has completed.  Faults inside a kernel surface at the
 *     caller's next synchronization with the stream.
 *   - Calls are stateless, thread-safe and deterministic: the same inputs
 *     give the same bits.  The only atomic is the integer maximum of the
 *     KV-scale recalibration, whose result does not depend on order.  The
 *     _ws calls use the caller's workspace as scratch for the call's
 *     duration only (one call at a time per workspace).
 * Errors (returned synchronously, after argument checks and the launch):
 *   - PRR_ERR_INVALID_ARG: a negative dimension, a dimension above
 *     2^31 - 1, or a NULL pointer for a non-empty operand;
 *   - PRR_ERR_UNSUPPORTED_SHAPE: a GEMM with K % 128 != 0 or K > 8388480
 *     (65535 blocks: the many-token kernel's 32-bit tile offsets), or an
 *     INT8 GEMM with K > 133143 (127^2 K could overflow its int32
 *     accumulator);
 *   - PRR_ERR_MISALIGNED: a pointer that is not 16-byte aligned;
 *   - PRR_ERR_NO_DEVICE: no HIP device is visible;
 *   - PRR_ERR_UNSUPPORTED_DEVICE: the current device is not gfx950;
 *   - PRR_ERR_HIP: the HIP runtime reported an error at launch.
 */
#ifndef PRR_H
#define PRR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PRR_ABI_VERSION 11

typedef enum prr_status {
  PRR_OK = 0,
  PRR_ERR_INVALID_ARG = 1,
  PRR_ERR_UNSUPPORTED_SHAPE = 2,
  PRR_ERR_MISALIGNED = 3,
  PRR_ERR_NO_DEVICE = 4,
  PRR_ERR_UNSUPPORTED_DEVICE = 5,
  PRR_ERR_HIP = 6
} prr_status;

/*
 * fp8_weight_block_quant -- FP8 e4m3 re-quantization of one bf16 weight in
 * 128 x 128 blocks (FP8-RL, abstract: repeated per-step quantization of the
 * changing policy weights; item (i): blockwise FP8).
 *   w_bf16  in   [N, K] bf16 bits, row-major (Wt layout).
 *   N, K         rows (output channels) and columns (input features), >= 0.
 *   w_fp8   out  [N, K] e4m3 codes, row-major.
 *   w_scale out  [ceil(N/128), ceil(K/128)] fp32, row-major: block (i, j)
 *                covers rows 128i.. and columns 128j.. of w_bf16.
 */
prr_status fp8_weight_block_quant(const uint16_t* w_bf16, int64_t N, int64_t K,
                                  uint8_t* w_fp8, float* w_scale,
                                  hipStream_t stream);

/*
 * fp8_weight_block_quant_into -- the same quantization of one shard of a
 * weight, written in place into the full weight's code and scale arrays:
 * the step that turns the bf16 shard a weight synchronization delivers into
 * the inference engine's FP8 weight (FP8-RL, abstract: the changing policy
 * weights are quantized again and synchronized into the inference engine
 * every step), chunk by chunk as the shard arrives.
 *   w_bf16   in   [rows, cols] bf16 bits, row stride ld_w elements.
 *   q_fp8    out  [rows, cols] e4m3 codes, row stride ld_q bytes.
 *   scale    out  [ceil(rows/128), ceil(cols/128)] fp32, row stride
 *                 ld_scale floats; block (i, j) covers rows 128i.. and
 *                 columns 128j.. of the shard.
 *   The shard is quantized as a matrix of its own (blocks anchored at its
 *   first row and column, partial blocks at its edges).  With q_fp8 and
 *   scale pointing at row 128a and column 128b of a full weight's arrays
 *   (ld_q = K, ld_scale = ceil(K/128)), the result is that part of
 *   fp8_weight_block_quant of the full weight: the blocks are the same.
 *   rows, cols >= 0; ld_w, ld_q >= cols; ld_scale >= ceil(cols/128)
 *   (PRR_ERR_INVALID_ARG otherwise); w_bf16 and q_fp8 16-byte aligned,
 *   scale 4-byte aligned (PRR_ERR_MISALIGNED otherwise).
 */
prr_status fp8_weight_block_quant_into(const uint16_t* w_bf16, int64_t rows, int64_t cols,
                                       int64_t ld_w, uint8_t* q_fp8, int64_t ld_q, float* scale,
                                       int64_t ld_scale, hipStream_t stream);

/*
 * fp8_weight_block_quant_multi / int8_weight_channel_quant_multi -- the
 * per-step re-quantization of several weights at once, e.g. every weight of
 * a decoder layer after a training step (FP8-RL, abstract: the policy
 * weights change every step and are quantized again every step), in one
 * launch: the same codes and scales, bit for bit, as
 * fp8_weight_block_quant / int8_weight_channel_quant called once per
 * weight.  One launch lets small weights (a k or v projection) share the
 * machine with large ones instead of paying a launch ramp each.
 *   jobs   host array of `count` descriptors, read during the call only
 *          (the library copies them into the launch): each names a whole
 *          weight w_bf16 [N, K] and its outputs, q (FP8: uint8 e4m3 codes;
 *          INT8: int8 codes) [N, K] and scale (FP8: [ceil(N/128),
 *          ceil(K/128)]; INT8: [N]) fp32, all row-major device memory.
 *   count  0 .. PRR_MAX_WEIGHT_JOBS (PRR_ERR_INVALID_ARG otherwise).
 *   Each job is checked as the single-weight call checks it (dimensions,
 *   NULL and 16-byte alignment of its pointers); a job with N == 0, or
 *   K == 0 for FP8, writes nothing (INT8 with K == 0 writes zero scales).
 *   Jobs must not overlap one another's outputs.  PRR_ERR_UNSUPPORTED_SHAPE
 *   when the jobs together exceed 2^31 - 1 work units.
 */
#define PRR_MAX_WEIGHT_JOBS 16
typedef struct prr_weight_job {
  const uint16_t* w_bf16;
  int64_t N, K;
  void* q;
  float* scale;
} prr_weight_job;
prr_status fp8_weight_block_quant_multi(const prr_weight_job* jobs, int64_t count,
                                        hipStream_t stream);
prr_status int8_weight_channel_quant_multi(const prr_weight_job* jobs, int64_t count,
                                           hipStream_t stream);

/*
 * fp8_act_token_quant -- FP8 e4m3 quantization of bf16 activations in
 * per-token groups of 128 consecutive input features (FP8-RL, abstract,
 * item (i): the "A8" of W8A8).
 *   a_bf16  in   [M, K] bf16 bits, row-major (token x feature).
 *   a_fp8   out  [M, K] e4m3 codes.
 *   a_scale out  [M, ceil(K/128)] fp32: group j of row m covers columns
 *                128j .. 128j+127 of that row.
 */
prr_status fp8_act_token_quant(const uint16_t* a_bf16, int64_t M, int64_t K,
                               uint8_t* a_fp8, float* a_scale,
                               hipStream_t stream);

/*
 * w8a8_block_gemm -- the FP8 W8A8 linear layer with block scales and bf16
 * output (FP8-RL, abstract, item (i)):
 *   C[m, n] = bf16( sum_kb a_scale[m, kb] * w_scale[n / 128, kb]
 *                   * sum_{k in kb} D(a_fp8[m, k]) * D(w_fp8[n, k]) )
 * with D the exact e4m3 value, fp32 accumulation and one RNE rounding to
 * bf16.  The result agrees with the fp64 evaluation of the same sum,
 * rounded once to bf16, within a relative Frobenius error of 1e-3.
 *   a_fp8 [M, K], a_scale [M, K/128]   as written by fp8_act_token_quant.
 *   w_fp8 [N, K], w_scale [ceil(N/128), K/128] as written by
 *                                      fp8_weight_block_quant.
 *   M, N >= 0; K >= 0 with K % 128 == 0 and K <= 8388480 (K == 0 writes
 *   +0.0).
 *   c_bf16 out [M, N] bf16 bits, row-major.
 */
prr_status w8a8_block_gemm(const uint8_t* a_fp8, const float* a_scale,
                           const uint8_t* w_fp8, const float* w_scale,
                           int64_t M, int64_t N, int64_t K, uint16_t* c_bf16,
                           hipStream_t stream);

/*
 * int8_weight_channel_quant -- INT8 re-quantization of one bf16 weight with
 * one scale per output channel (FlashRL article: INT8 rollout with
 * per-step quantization of the updated weights; granularity fixed here).
 *   w_bf16  in   [N, K] bf16 bits (Wt layout).
 *   w_i8    out  [N, K] int8 codes.
 *   w_scale out  [N] fp32: row n's scale, over all K of that row.
 */
prr_status int8_weight_channel_quant(const uint16_t* w_bf16, int64_t N,
                                     int64_t K, int8_t* w_i8, float* w_scale,
                                     hipStream_t stream);

/*
 * int8_act_token_quant -- dynamic INT8 quantization of bf16 activations
 * with one scale per token over the whole K (FlashRL article: INT8
 * rollout; granularity fixed here).
 *   a_bf16  in   [M, K] bf16 bits.
 *   a_i8    out  [M, K] int8 codes.
 *   a_scale out  [M] fp32.
 */
prr_status int8_act_token_quant(const uint16_t* a_bf16, int64_t M, int64_t K,
                                int8_t* a_i8, float* a_scale,
                                hipStream_t stream);

/*
 * w8a8_int8_channel_gemm -- the INT8 W8A8 linear layer (FlashRL article):
 *   acc[m, n] = sum_k a_i8[m, k] * w_i8[n, k]     (exact, int32)
 *   C[m, n]   = bf16(acc[m, n] * a_scale[m] * w_scale[n])
 * evaluated in fp32 and rounded once to bf16; agrees with the fp64
 * evaluation rounded once to bf16 within a relative Frobenius error of 1e-3.
 *   a_i8 [M, K], a_scale [M]; w_i8 [N, K], w_scale [N];
 *   K % 128 == 0 and K <= 133143; c_bf16 out [M, N].
 */
prr_status w8a8_int8_channel_gemm(const int8_t* a_i8, const float* a_scale,
                                  const int8_t* w_i8, const float* w_scale,
                                  int64_t M, int64_t N, int64_t K,
                                  uint16_t* c_bf16, hipStream_t stream);

/*
 * w8a8_gemm_workspace_size / w8a8_block_gemm_ws / w8a8_int8_channel_gemm_ws
 * -- the two GEMMs above with an optional caller-owned workspace, for
 * decode-sized batches (M <= 64) of layers with few output channels or long
 * K (e.g. a down projection, N 5120 x K 27648), where one workgroup per
 * 16-channel strip over all of K leaves CUs idle or cannot hold the
 * activations, and for many-token batches (M > 128) of long-K layers
 * (K >= 8192) whose output tiles leave a last, partial round on the CUs.
 * With the workspace the call splits K into S slices (for many tokens,
 * those of the last round's tile columns only), writes fp32 partial sums
 * (INT8: int32 accumulators) to it and adds the slices in a fixed order
 * (bitwise repeatable; same definition and tolerance as the one-pass call;
 * INT8 results are identical to the one-pass call's).  Callers that cannot
 * provide one use the calls above.
 *   w8a8_gemm_workspace_size: *bytes = the workspace the _ws calls use for
 *       this shape on the current device (S x M x N x 4 for decode batches,
 *       S x M x the split columns x 4 for many tokens; 0 = no split, the
 *       _ws call runs the one-pass kernels).  Same for FP8 and INT8.
 *   workspace: device memory, 16-byte aligned, not shared with a call in
 *       flight on another stream; NULL or workspace_bytes below the size
 *       -> the one-pass kernels (never an error).  The library does not
 *       keep the pointer.
 *   Other arguments and errors as w8a8_block_gemm / w8a8_int8_channel_gemm;
 *   workspace_bytes < 0 -> PRR_ERR_INVALID_ARG.
 */
prr_status w8a8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, int64_t* bytes);
prr_status w8a8_block_gemm_ws(const uint8_t* a_fp8, const float* a_scale, const uint8_t* w_fp8,
                              const float* w_scale, int64_t M, int64_t N, int64_t K,
                              uint16_t* c_bf16, void* workspace, int64_t workspace_bytes,
                              hipStream_t stream);
prr_status w8a8_int8_channel_gemm_ws(const int8_t* a_i8, const float* a_scale,
                                     const int8_t* w_i8, const float* w_scale, int64_t M,
                                     int64_t N, int64_t K, uint16_t* c_bf16, void* workspace,
                                     int64_t workspace_bytes, hipStream_t stream);

/*
 * w8a8_block_gemm_scratch -- w8a8_block_gemm_ws for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the same definition, arguments,
 * kernels and tolerance, with the split-K partial sums in the library's own
 * static device array of 16 MiB (one per device, kept until the process
 * ends) instead of a caller workspace.  The call itself allocates nothing.
 * Every call on a device shares that device's array: calls that overlap on
 * one device (on two streams, or from two threads) race and give undefined
 * results; calls in order on one stream are safe.  A shape whose split
 * needs more than 16 MiB (S x M x N x 4 bytes, as
 * w8a8_gemm_workspace_size reports) returns PRR_ERR_UNSUPPORTED_SHAPE
 * without launching; a shape with no split runs the one-pass kernels.
 * Decode batches (M <= 64) split exactly as w8a8_block_gemm_ws does, with
 * its results bit for bit; many-token batches (M > 128) run the one-pass
 * kernels, w8a8_block_gemm's results (the workspace call's split of their
 * last round needs slabs of tens of MB).
 */
prr_status w8a8_block_gemm_scratch(const uint8_t* a_fp8, const float* a_scale,
                                   const uint8_t* w_fp8, const float* w_scale, int64_t M,
                                   int64_t N, int64_t K, uint16_t* c_bf16, hipStream_t stream);

/*
 * w8a8_block_gemm_grouped -- the FP8 W8A8 linear layer of a mixture of
 * experts (FP8-RL, abstract: the FP8 rollout stack covers dense and MoE
 * models), for decode-sized groups: one launch for every expert.
 *   a_fp8 [M, K], a_scale [M, K/128]  token rows sorted by expert, as
 *                       written by fp8_act_token_quant.
 *   w_fp8 [E, N, K], w_scale [E, ceil(N/128), K/128]  each expert's weight
 *                       as written by fp8_weight_block_quant.
 *   expert_offsets [E + 1] int64, device memory: rows offsets[e] ..
 *                       offsets[e+1] - 1 go to expert e (non-decreasing;
 *                       values are clamped into [0, M], so rows before
 *                       offsets[0] or from offsets[E] on are not written).
 *   max_rows_per_expert a bound on the rows of any expert, used only to
 *                       choose the register tiling (<= 16, <= 32, else 64
 *                       rows); groups above 64 rows are processed in 64-row
 *                       chunks, each of which reads the expert's weight.
 *   c_bf16 out [M, N]   each group's rows are w8a8_block_gemm of the group
 *                       with its expert's weight (same definition and
 *                       tolerance).
 *   E, M, N >= 0; K > 0 with K % 128 == 0 and K <= 6144 (PRR_ERR_
 *   UNSUPPORTED_SHAPE beyond: the activations of a 64-row chunk must fit
 *   in registers; 8192 when max_rows_per_expert <= 32).
 */
prr_status w8a8_block_gemm_grouped(const uint8_t* a_fp8, const float* a_scale,
                                   const uint8_t* w_fp8, const float* w_scale,
                                   const int64_t* expert_offsets, int64_t E, int64_t M,
                                   int64_t N, int64_t K, int64_t max_rows_per_expert,
                                   uint16_t* c_bf16, hipStream_t stream);

/*
 * fp8_kv_scale_recalibrate -- per-step recalibration of one FP8 KV-cache
 * scale (FP8-RL, abstract, item (ii): the Q/K/V scales are recalibrated at
 * every step; one scale per tensor is this library's reading).  Call once
 * per tensor (K, V, and Q for an FP8 attention read path) per step.
 *   x_bf16 in   [T, C] bf16 bits: a calibration batch of the tensor, e.g.
 *               the K projection output (C = kv_heads x head_dim).  May be
 *               NULL when T x C == 0.
 *   T, C        >= 0.
 *   scale  out  one fp32: s = fl32(max |x| / 448) over all T x C values
 *               (+0.0 for an all-zero or empty tensor).  The word is the
 *               reduction's accumulator while the call's kernels run, so
 *               nothing may read it before they complete.
 */
prr_status fp8_kv_scale_recalibrate(const uint16_t* x_bf16, int64_t T, int64_t C,
                                    float* scale, hipStream_t stream);

/*
 * fp8_kv_cache_write -- quantize-on-write of new K or V rows into an FP8
 * cache (FP8-RL, abstract, item (ii)).
 *   kv_bf16      in     [T, C] bf16 bits, one row per new token.
 *   slot_mapping in     [T] int64: the cache row of each token.  A slot
 *                       outside [0, num_slots) -- negative for a padding
 *                       token -- skips that token.  Slots in range must be
 *                       distinct (otherwise which token lands is undefined).
 *   scale        in     one fp32 in device memory, e.g. written by
 *                       fp8_kv_scale_recalibrate.  Codes are
 *                       E4M3_saturating_RNE(fl32(x / s)): values beyond the
 *                       calibrated range saturate to +-448; s = 0 writes the
 *                       signed zeros of x.
 *   cache        in/out [num_slots, C] e4m3 codes; rows no token maps to
 *                       are not touched.
 *   T, C, num_slots >= 0; T == 0, C == 0 or num_slots == 0 is a no-op.
 */
prr_status fp8_kv_cache_write(const uint16_t* kv_bf16, const int64_t* slot_mapping,
                              int64_t T, int64_t C, const float* scale, uint8_t* cache,
                              int64_t num_slots, hipStream_t stream);

/*
 * fp8_kv_cache_write_recalibrate -- one step of the FP8 KV cache (FP8-RL,
 * abstract, item (ii)) in one pass over the step's new rows: they are
 * written into the cache with the scale an earlier batch calibrated,
 * exactly as fp8_kv_cache_write(kv_bf16, slot_mapping, T, C, scale, cache,
 * num_slots), and the next step's scale is recalibrated from the same rows,
 * exactly as fp8_kv_scale_recalibrate(kv_bf16, T, C, new_scale).  The two
 * separate calls read the rows twice; this one reads them once.
 *   kv_bf16, slot_mapping, scale, cache, T, C, num_slots: as
 *                fp8_kv_cache_write (the write is a no-op when num_slots
 *                is 0; kv_bf16 and slot_mapping may be NULL when T x C is
 *                0, cache when num_slots is 0).
 *   new_scale  out  one fp32: fl32(max |kv| / 448) over all T x C values,
 *                every row counted whether or not its slot is in range
 *                (+0.0 for an all-zero or empty batch).  Written by the
 *                call's last kernel, after every read of `scale`, so it may
 *                be the `scale` word itself (the scale updated in place).
 *   workspace  device memory, 16-byte aligned, of workspace_bytes >=
 *                PRR_KV_RECAL_WORKSPACE_BYTES (else PRR_ERR_INVALID_ARG):
 *                the workgroups' partial maxima, for the call's duration
 *                only (one call at a time per workspace; no clearing
 *                needed).  May be NULL when T x C == 0.
 */
#define PRR_KV_RECAL_WORKSPACE_BYTES 8192
prr_status fp8_kv_cache_write_recalibrate(const uint16_t* kv_bf16,
                                          const int64_t* slot_mapping, int64_t T,
                                          int64_t C, const float* scale, uint8_t* cache,
                                          int64_t num_slots, float* new_scale,
                                          void* workspace, int64_t workspace_bytes,
                                          hipStream_t stream);

/*
 * fp8_kv_cache_write_recalibrate_multi -- fp8_kv_cache_write_recalibrate
 * for up to PRR_MAX_KV_JOBS tensors of one step that share the slot mapping
 * (K and V: FP8-RL, abstract, item (ii)), in one launch over all of their
 * rows and one over their partial maxima; each job's results are those of
 * the single call.
 *   jobs   host array of `count` prr_kv_job: kv_bf16 [T, C], the scale it is
 *          written with, its cache [num_slots, C], its new_scale (which may
 *          be its own scale word).  The new_scale words must be distinct
 *          (PRR_ERR_INVALID_ARG otherwise); caches and the other jobs'
 *          scales must not overlap what another job writes.
 *   count  0 .. PRR_MAX_KV_JOBS (0: nothing is done).
 *   slot_mapping, T, C, num_slots: shared, as fp8_kv_cache_write.
 *   workspace  count x PRR_KV_RECAL_WORKSPACE_BYTES bytes at least, 16-byte
 *          aligned (job j's partials at byte j x PRR_KV_RECAL_WORKSPACE_BYTES),
 *          for the call's duration only; may be NULL when T x C == 0.
 */
#define PRR_MAX_KV_JOBS 16
typedef struct prr_kv_job {
  const uint16_t* kv_bf16;
  const float* scale;
  uint8_t* cache;
  float* new_scale;
} prr_kv_job;
prr_status fp8_kv_cache_write_recalibrate_multi(const prr_kv_job* jobs, int64_t count,
                                                const int64_t* slot_mapping, int64_t T,
                                                int64_t C, int64_t num_slots, void* workspace,
                                                int64_t workspace_bytes, hipStream_t stream);

/*
 * fp8_kv_decode_attention -- the read side of the FP8 KV cache (FP8-RL,
 * abstract, item (ii): FP8 KV cache with per-step Q/K/V scales): attention
 * of one new token per sequence over its cached tokens.  The pages give no
 * kernel; this library's reading: the query is quantized per tensor with
 * q_scale (the cache's e4m3 encode); score of cached token t for query head
 * h: s_q s_k softmax_scale (q^_h . k^_t) against cache head h / (Hq / Hkv);
 * softmax over the sequence's seq_lens[b] tokens; output s_v sum_t p_t v^_t
 * rounded to bf16.  fp32 arithmetic; the output is judged like a GEMM
 * (relative Frobenius error <= 1e-3 against the fp64 definition).
 *   q_bf16      in  [B, Hq, D] bf16 bits: the new token's queries.
 *   q_scale, k_scale, v_scale  in  one fp32 each, device memory (e.g. from
 *                   fp8_kv_scale_recalibrate of Q, K and V).
 *   k_cache, v_cache  in  [num_slots, Hkv * D] e4m3 codes (e.g. written by
 *                   fp8_kv_cache_write); the new token's K and V are
 *                   expected in the cache already.
 *   block_table in  [B, max_blocks] int32: token t of sequence b is in slot
 *                   block_table[b][t / page] * page + t % page.  A token
 *                   whose slot is negative or >= num_slots is skipped.
 *   seq_lens    in  [B] int32: cached tokens per sequence (clamped to
 *                   [0, max_blocks * page]); 0 writes zeros.
 *   softmax_scale   finite (typically 1 / sqrt(D)).
 *   out_bf16    out [B, Hq, D].
 *   D must be 128, Hq / Hkv (a whole number) at most 8 and page at most
 *   2^20 (PRR_ERR_UNSUPPORTED_SHAPE otherwise); Hkv, page and max_blocks
 *   >= 1 when B x Hq > 0.
 */
prr_status fp8_kv_decode_attention(const uint16_t* q_bf16, const float* q_scale,
                                   const uint8_t* k_cache, const uint8_t* v_cache,
                                   const float* k_scale, const float* v_scale,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page,
                                   int64_t max_blocks, int64_t num_slots, float softmax_scale,
                                   uint16_t* out_bf16, hipStream_t stream);

/*
 * fp8_kv_decode_attention_workspace_size / fp8_kv_decode_attention_ws -- the
 * call above with an optional caller-owned workspace (same definition,
 * arguments, errors and tolerance).  With it the batch's cached tokens,
 * sequence after sequence, are cut into one equal range per compute unit; a
 * workgroup reads whole cache rows (every KV head of a token) over its
 * range and leaves a partial softmax state (unnormalized output, running
 * maximum and sum per query head) in the workspace for each sequence its
 * range meets; a second kernel combines the partial states of each
 * sequence in a fixed order (bitwise repeatable) and rounds once to bf16.
 * The one-pass call gives each (sequence, KV head) a workgroup of its own,
 * which reads 128 bytes of every Hkv x 128-byte cache row and leaves CUs
 * idle when the batch is small.
 *   fp8_kv_decode_attention_workspace_size: *bytes = the workspace the _ws
 *       call uses for B sequences of Hq query heads over Hkv KV heads of D
 *       on the current device (0: the shape takes the one-pass kernel:
 *       D != 128, B > 2048, or Hkv > 8).
 *   workspace: device memory, 16-byte aligned, not shared with a call in
 *       flight on another stream; NULL or workspace_bytes below the size ->
 *       the one-pass kernel (never an error).  The library does not keep
 *       the pointer.  workspace_bytes < 0 -> PRR_ERR_INVALID_ARG.
 */
prr_status fp8_kv_decode_attention_workspace_size(int64_t B, int64_t Hq, int64_t Hkv, int64_t D,
                                                  int64_t* bytes);
prr_status fp8_kv_decode_attention_ws(const uint16_t* q_bf16, const float* q_scale,
                                      const uint8_t* k_cache, const uint8_t* v_cache,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int64_t B, int64_t Hq, int64_t Hkv, int64_t D, int64_t page,
                                      int64_t max_blocks, int64_t num_slots, float softmax_scale,
                                      uint16_t* out_bf16, void* workspace,
                                      int64_t workspace_bytes, hipStream_t stream);

/*
 * tis_token_weights -- token-level importance weights for correcting the
 * mismatch between the rollout policy (e.g. an FP8 rollout engine) and the
 * trainer's policy (FP8-RL, abstract, item (iii): token-level TIS/MIS
 * rollout correction; FlashRL article, section on the rollout-training
 * mismatch: truncated importance sampling).  The pages print no formula;
 * this library's reading, per response token t of sequence b:
 *   d   = fl32(logp_train - logp_rollout)          (binary32 subtraction)
 *   over = d > fl32(ln cap)                         (ln in fp64, rounded once)
 *   PRR_IS_TRUNCATE (TIS): w = over ? cap : expf(d)     (= min(ratio, cap))
 *   PRR_IS_MASK     (MIS): w = over ? 0   : expf(d)     (token left out)
 *   padding (mask 0): w = 0, counted in no statistic; its log-probabilities
 *   are never used (they may hold anything, NaN included).
 *   logp_train, logp_rollout in [B, T] fp32: log-probability of each sampled
 *                       token under the trainer's / the rollout engine's
 *                       policy (finite on response tokens).
 *   mask       in  [B, T] uint8: nonzero = response token.
 *   cap        truncation constant C > 0 (+inf: plain importance ratios).
 *   weights    out [B, T] fp32.  expf(d) is within 2 ulp of exp(d).
 *   row_stats  out [B, 4] fp32 or NULL: per sequence (valid tokens, tokens
 *                  over the cap, sum of w, sum of logp_rollout - logp_train);
 *                  counts are exact (T <= 2^24), the sums are fp32 added in
 *                  a fixed order (bitwise repeatable).  The last one divided
 *                  by the first is the sample estimate of KL(rollout ||
 *                  trainer).
 *   totals     out [4] fp64 or NULL: the sums over all sequences of
 *                  row_stats (fixed order); requires row_stats when B > 0.
 *   B, T >= 0; T > 2^24 -> PRR_ERR_UNSUPPORTED_SHAPE; cap not > 0 (NaN
 *   included), an unknown mode, or totals without row_stats ->
 *   PRR_ERR_INVALID_ARG.  T % 4 == 0 takes the vector path.
 */
#define PRR_IS_TRUNCATE 0
#define PRR_IS_MASK 1
prr_status tis_token_weights(const float* logp_train, const float* logp_rollout,
                             const uint8_t* mask, int64_t B, int64_t T, float cap, int mode,
                             float* weights, float* row_stats, double* totals,
                             hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* prr_status_string(prr_status status);

/* PRR_ABI_VERSION of the library that is loaded. */
int prr_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PRR_H */

// Decode attention over the FP8 KV cache ("FP8-RL: A Practical and Stable
// Low-Precision Stack for LLM Reinforcement Learning", abstract, item (ii):
// FP8 KV cache with per-step Q/K/V scales).  One new token per sequence;
// query head h reads cache head h / (Hq / Hkv).  The query is quantized with
// its per-tensor scale by the library's e4m3 encoder; score of cached token
// t: s_q s_k c (q^ . k^_t); softmax over the sequence's tokens; output
// s_v sum_t p_t v^_t, rounded once to bf16.
//
// Bound by HBM: every cached token costs 2 x 128 bytes per KV head (its K
// and V codes) against ~5 flops per byte for a group of 5 query heads.
//
// Two launch forms share the token loop's design: the one-pass kernel
// (no workspace; described here) and, with a caller workspace, a split of
// the batch's tokens over the CUs (described before its kernels below).
//
//  * One 512-thread workgroup per (sequence, KV head), taken longest
//    sequence first (ranked in-kernel from the lengths, up to 256
//    sequences); wave w takes iterations w, w + 8, ... of the sequence, 32
//    tokens (two tiles of 16) an iteration, and keeps the next iteration's
//    K and V loads in flight behind the current one's math.
//  * Q K^T on the matrix cores in bf16: e4m3 -> bf16 is exact, and the bf16
//    16x16x32 instruction sums its products to fp32 accuracy, while the
//    e4m3 instructions of gfx950 keep only ~13 bits inside a dot product
//    (measured: errors up to 2e-4 of the sum of |products|), which the
//    softmax would turn into output errors well above a bf16 rounding.  One
//    tile of 16 tokens against the group's query heads (rows past G zero) is
//    four instructions, with no cross-lane reduction.
//  * Online softmax in the base-2 domain (scores carry log2 e), updated once
//    per iteration per head.  P V on the matrix cores in fp16: each weight
//    is split into fp16 hi + lo parts (~2^-21 relative together), V is
//    decoded exactly from e4m3 to fp16 after a transposing LDS read of the
//    wave's token-major V tile.  The 8 waves are combined through LDS.
//  * The sequence's block-table row is staged in LDS (2048 pages at a
//    time) as a byte base and a count of valid slots per page.  Loads are
//    branch-free: an absent token (past the length, or its slot outside the
//    cache) reads cache row 0 and is masked out of the softmax.
#include "launch.h"
#include "prr_device.h"

namespace prr {

constexpr int kAttThreads = 512;
constexpr int kAttWaves = kAttThreads / 64;
constexpr int kAttD = 128;            // head dimension
constexpr int kAttIter = 32;          // tokens of a wave iteration (two tiles of 16)
constexpr int kAttTablePages = 2048;  // block-table entries staged at a time
constexpr int kAttOrderMax = 256;     // sequences ordered by length in-kernel (at most)
constexpr int kAttVRow = 144;         // LDS bytes a token of the V tile (128 + bank skew)
constexpr int kAttVTile = kAttIter * kAttVRow;
constexpr float kAttWeightExp = 14.f; // weights scaled by 2^14 (fp16 range)
constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));

// Eight e4m3 codes -> eight bf16 values (exact: every e4m3 value, subnormals
// included, is a bf16 value), in code order.
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  const uint4 r = make_uint4(
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)));
  return __builtin_bit_cast(v8bf, r);
}

// x / d for x < 2^24 and a quotient below 2^6 (x at most 32 past a
// multiple of d): one float product, corrected by one step either way.
__device__ __forceinline__ uint32_t small_div(uint32_t x, uint32_t d, float inv_d) {
  uint32_t qt = (uint32_t)((float)x * inv_d);
  const int32_t rem = (int32_t)(x - qt * d);
  if (rem < 0) --qt;
  else if (rem >= (int32_t)d) ++qt;
  return qt;
}

// Eight e4m3 codes (a 64-bit pair) -> eight fp16 values (exact: every e4m3
// value, subnormals included, is an fp16 value), in code order.
__device__ __forceinline__ v8h e4m3x8_to_f16(uint32_t lo, uint32_t hi) {
  const uint4 r = make_uint4(
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false)),
      __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true)));
  return __builtin_bit_cast(v8h, r);
}

// The token loop of the split kernel, over one staged chunk of a sequence,
// for one KV head: the
// wave takes iterations it_first, it_first + it_step, ... of 32 tokens over
// the chunk's ntok tokens, updating its online-softmax state (m, l, acc) for
// the G query heads of lane row r.  tbase / tlim: the staged pages (byte
// base of the page's first row, slots of the page inside the cache).
template <int G>
__device__ __forceinline__ void att_chunk(const int64_t* tbase, const int32_t* tlim, int ntok,
                                          uint32_t cb, int page, float inv_page,
                                          uint32_t row_bytes, const uint8_t* kbase,
                                          const uint8_t* vbase, uint8_t* vt,
                                          const uint8_t* tr_src, const uint4* qrow, float cs,
                                          int it_first, int it_step, int g, int r, float& m,
                                          float& l, v4f (&acc)[8]) {
  const int iters = (ntok + kAttIter - 1) / kAttIter;
  // Token k of iteration it is token 32 it + k of the chunk, at position
  // cb + 32 it + k from the first staged page: page pi0 + (off0 + k) / page
  // of the staged table, all in 32 bits (a chunk holds at most 2^30
  // tokens).  A token that is absent (past the length, or its slot outside
  // the cache) reads row 0 of the cache (there is one) and is masked.  Lane
  // (g, r) locates token 16 tile + r.
  auto locate = [&](int it, uint64_t at[2], bool ok[2]) {
    const uint32_t rel0 = (uint32_t)it * kAttIter, pos0 = cb + rel0;
    const uint32_t pi0 = pos0 / (uint32_t)page, off0 = pos0 - pi0 * (uint32_t)page;
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const int k = 16 * tile + r;
      const bool in = (int)rel0 + k < ntok;
      const uint32_t off = off0 + (uint32_t)k;
      const uint32_t qp = small_div(off, (uint32_t)page, inv_page);
      const uint32_t pi = in ? pi0 + qp : 0;
      const uint32_t o = off - qp * (uint32_t)page;
      // (pi is in range either way; the empty asm keeps the compiler from
      // moving the reads under a branch on ok)
      int32_t lim = tlim[pi];
      int64_t base = tbase[pi];
      asm volatile("" : "+v"(lim), "+v"(base));
      ok[tile] = in & ((int32_t)o < lim);
      at[tile] = ok[tile] ? (uint64_t)base + (uint64_t)o * row_bytes : 0;
    }
  };
  auto load_k = [&](const uint64_t at[2], uint4 kx[2][2]) {
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint4* kp = reinterpret_cast<const uint4*>(kbase + at[tile]);
      kx[tile][0] = kp[0];
      kx[tile][1] = kp[1];
    }
  };
  auto load_v = [&](const uint64_t at[2], uint4 vx[2][2]) {
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      const uint4* vp = reinterpret_cast<const uint4*>(vbase + at[tile]);
      vx[tile][0] = vp[0];
      vx[tile][1] = vp[1];
    }
  };
  // Each wave keeps the next iteration's loads in flight behind this
  // one's work: its K loads go out once Q K^T has consumed the current
  // K, its V loads once the current V is in the LDS tile (same registers).
  uint64_t at[2];
  bool ok[2];
  uint4 kx[2][2], vx[2][2];
  if (it_first < iters) {
    locate(it_first, at, ok);
    load_k(at, kx);
    load_v(at, vx);
  }
  for (int it = it_first; it < iters; it += it_step) {
    const bool more = it + it_step < iters;
    uint64_t at_n[2] = {0, 0};
    bool ok_n[2] = {false, false};
    if (more) locate(it + it_step, at_n, ok_n);
    uint64_t okm[2];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) okm[tile] = __ballot(ok[tile]) & 0xFFFF;  // bit j: token 16 tile + j
    // Scores (base 2): lane (g, r) gets tokens 16 tile + 4 g + i of head r.
    float sc[2][4];
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      v4f d = {0.f, 0.f, 0.f, 0.f};
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kx[tile][0].x, kx[tile][0].y),
                                                  __builtin_bit_cast(v8bf, qrow[0]), d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kx[tile][0].z, kx[tile][0].w),
                                                  __builtin_bit_cast(v8bf, qrow[1]), d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kx[tile][1].x, kx[tile][1].y),
                                                  __builtin_bit_cast(v8bf, qrow[2]), d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kx[tile][1].z, kx[tile][1].w),
                                                  __builtin_bit_cast(v8bf, qrow[3]), d, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[tile][i] = ((okm[tile] >> (4 * g + i)) & 1) ? d[i] * cs : -__builtin_inff();
    }
    if (more) load_k(at_n, kx);
    // The V tile to LDS, token-major (read back transposed below; the
    // tile is this wave's own and its LDS operations complete in order).
    // An absent token's weight is 0; its V is zeroed so that whatever row
    // 0 holds cannot turn 0 into NaN.
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      uint4* dst = reinterpret_cast<uint4*>(vt + (16 * tile + r) * kAttVRow + 32 * g);
      dst[0] = ok[tile] ? vx[tile][0] : make_uint4(0, 0, 0, 0);
      dst[1] = ok[tile] ? vx[tile][1] : make_uint4(0, 0, 0, 0);
    }
    if (more) load_v(at_n, vx);
#pragma unroll
    for (int tile = 0; tile < 2; ++tile) {
      at[tile] = at_n[tile];
      ok[tile] = ok_n[tile];
    }
    float mi = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                     fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
    mi = fmaxf(mi, __shfl_xor(mi, 16, 64));
    mi = fmaxf(mi, __shfl_xor(mi, 32, 64));
    const float mn = fmaxf(m, mi);
    // (every token so far skipped: mn = -inf; subtract 0 so that the
    // weights and alpha come out 0 rather than NaN)
    const float mref = (mn == -__builtin_inff() ? 0.f : mn) - kAttWeightExp;
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
    // Weights as fp16 pairs: p = hi + lo to ~2^-21 relative.
    float ps = 0.f;
    _Float16 wh[8], wl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float pv = __builtin_amdgcn_exp2f(sc[e >> 2][e & 3] - mref);
      ps += pv;
      wh[e] = (_Float16)pv;
      wl[e] = (_Float16)(pv - (float)wh[e]);
    }
    const v8h ph = {wh[0], wh[1], wh[2], wh[3], wh[4], wh[5], wh[6], wh[7]};
    const v8h pl = {wl[0], wl[1], wl[2], wl[3], wl[4], wl[5], wl[6], wl[7]};
    ps += __shfl_xor(ps, 16, 64);
    ps += __shfl_xor(ps, 32, 64);
    // (alpha = 0 on the first tokens: m was -inf; mn = -inf as well gives
    // NaN, where l and the outputs are still 0)
    const float a = mn == -__builtin_inff() ? 1.f : alpha;
    l = l * a + ps;
    if (__ballot(a != 1.f)) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] *= a;
    }
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) v2i*)(tr_src + 16 * j));
      const v8h vf = e4m3x8_to_f16((uint32_t)t.x, (uint32_t)t.y);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph, acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl, acc[j], 0, 0, 0);
    }
    asm volatile("" ::: "memory");
  }
}

// (This kernel keeps its own copy of the token loop: called through
// att_chunk it measured ~4% slower on the 32B batch, the compiler placing
// its waits differently.)
template <int G>
__global__ __launch_bounds__(kAttThreads) void fp8_decode_attention_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k_cache, const uint8_t* __restrict__ v_cache,
    const float* __restrict__ k_scale, const float* __restrict__ v_scale,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hq,
    int Hkv, int page, int max_blocks, int64_t num_slots, float softmax_scale,
    uint16_t* __restrict__ out) {
  typedef float Part[G][kAttD + 2];
  static_assert(sizeof(Part) * kAttWaves <= kAttWaves * kAttVTile, "partials fit the V tiles");
  __shared__ int64_t tbase[kAttTablePages];        // byte offset of a staged page's first row
  __shared__ int32_t tlim[kAttTablePages];         // its slots inside the cache (0: skipped)
  // Per-wave V tile of an iteration, token-major (kAttVRow bytes a token);
  // after the token loop the same space holds the waves' partial results.
  __shared__ __attribute__((aligned(16))) uint8_t vtile[kAttWaves * kAttVTile];
  __shared__ uint4 qsh[16 * 4 * 4];                 // query operand fragments (bf16)
  __shared__ int32_t pick;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int B = (int)(gridDim.x / Hkv);
  const int kvh = blockIdx.x % Hkv;
  const int64_t n_cap = (int64_t)max_blocks * page;
  auto length = [&](int bb) -> int64_t {
    const int64_t v = seq_lens[bb];
    return min(v < 0 ? (int64_t)0 : v, n_cap);
  };
  // Longest sequences first: workgroup i serves the sequence of rank i / Hkv
  // in order of decreasing length (ties by index), so that the work left
  // for the last workgroups to start is the shortest.  The ranks are a
  // permutation, so exactly one thread finds the target.
  int b = (int)(blockIdx.x / Hkv);
  if (B <= kAttOrderMax) {
    const int64_t* lens = tbase;                   // staging space until the table is loaded
    for (int e = tid; e < B; e += kAttThreads) tbase[e] = length(e);
    __syncthreads();
    for (int j = tid; j < B; j += kAttThreads) {
      const int64_t lj = lens[j];
      int rank = 0;
      for (int i = 0; i < B; ++i) rank += (lens[i] > lj) || (lens[i] == lj && i < j);
      if (rank == b) pick = j;
    }
    __syncthreads();
    b = pick;
  }
  // Lane (g, r), in the layout of the 16x16x32 instructions:
  //  * Q K^T (bf16): row r = token r of a 16-token tile (first operand) or
  //    query head r (second operand, zero past the group), dimensions
  //    [32 g, 32 g + 32) as 4 slices of 8; results: tokens 4 g .. 4 g + 3
  //    of head r.  K and V of token r are loaded by the same lanes.
  //  * P V (fp16), summed over the iteration's 32 tokens: k-slot e of lane
  //    (g, .) is token 16 (e / 4) + 4 g + e % 4, so the probabilities stay
  //    where Q K^T left them (second operand, row r = head r); the first
  //    operand, row r = dimension 16 j + r, is read from the V tile by a
  //    transposing LDS load; results: dimensions 16 j + 4 g .. 16 j + 4 g + 3
  //    of head r.
  const int g = lane >> 4, r = lane & 15;
  const uint32_t row_bytes = (uint32_t)Hkv * kAttD;
  const uint8_t* kbase = k_cache + (int64_t)kvh * kAttD + 32 * g;
  const uint8_t* vbase = v_cache + (int64_t)kvh * kAttD + 32 * g;
  uint8_t* vt = vtile + wave * kAttVTile;
  // The transposing load: lane (g, s) names 8 bytes, and lane (g, r) gets
  // byte r % 8 of the bytes named by lanes (g, 2 e + r / 8), e = 0 .. 7.  So
  // lane (g, s) names dimensions 16 j + 8 (s % 2) .. + 8 of token-slot
  // e = s / 2.
  const int tr_tok = 16 * (r >> 3) + 4 * g + ((r >> 1) & 3);
  const uint8_t* tr_src = vt + tr_tok * kAttVRow + 8 * (r & 1);
  uint16_t* ob = out + ((int64_t)b * Hq + (int64_t)kvh * G) * kAttD;

  // (no cache slots: every token is skipped)
  const int64_t n = num_slots > 0 ? length(b) : 0;
  if (n == 0) {
    for (int e = tid; e < G * kAttD; e += kAttThreads) ob[e] = 0;
    return;
  }

  // The group's query heads, quantized with s_q and decoded to bf16 (exact),
  // kept in LDS in the second operand's layout (row r = head r, zero past
  // the group; slice j of lane (g, r) = dimensions 32 g + 8 j .. + 8) and
  // read where used, which keeps 16 registers free for the loads in flight.
  const float sq = *q_scale;
  if (wave == 0) {
    const BlockDiv dq = block_div(sq);
    const uint16_t* qh = q + ((int64_t)b * Hq + (int64_t)kvh * G + r) * kAttD + 32 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 w = make_uint4(0, 0, 0, 0);
      if (r < G) {
        const uint2 c = e4m3_chunk_any<true>(*reinterpret_cast<const uint4*>(qh + 8 * j), sq, dq);
        w = __builtin_bit_cast(uint4, e4m3x8_to_bf16(c.x, c.y));
      }
      qsh[(r * 4 + g) * 4 + j] = w;
    }
  }
  const uint4* qrow = &qsh[(r * 4 + g) * 4];
  // Score scale in the base-2 domain.  Weights are 2^(s - m + 14), in
  // [0, 2^14], so that their fp16 halves stay clear of the subnormals; the
  // factor cancels in O / L.
  const float cs = sq * (*k_scale) * softmax_scale * kLog2e;
  const float sv = *v_scale;
  const float inv_page = 1.0f / (float)page;

  float m = -__builtin_inff(), l = 0.f;              // head r (equal in the 4 lanes of r)
  v4f acc[8];                                        // dims 16 j + 4 g + e' of head r
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};

  const int32_t* trow = block_table + (int64_t)b * max_blocks;
  // (at most 2^30 tokens a chunk: token positions stay in 32 bits)
  const int64_t chunk_tokens = (int64_t)min(kAttTablePages, (1 << 30) / page) * page;
  for (int64_t c0 = 0; c0 < n; c0 += chunk_tokens) {
    const int64_t c1 = min(n, c0 + chunk_tokens);
    const int p0 = (int)(c0 / page);
    const int np = (int)((c1 - c0 + page - 1) / page);
    __syncthreads();                                   // previous readers of the table are done
    for (int e = tid; e < np; e += kAttThreads) {
      const int64_t pid = trow[p0 + e];
      const int64_t first = pid * page;
      const int64_t lim = pid < 0 ? 0 : min((int64_t)page, max((int64_t)0, num_slots - first));
      tlim[e] = (int32_t)lim;
      tbase[e] = lim > 0 ? first * row_bytes : 0;
    }
    __syncthreads();
    const int iters = (int)((c1 - c0 + kAttIter - 1) / kAttIter);
    const int ntok = (int)(c1 - c0);
    // Token k of iteration it is token 32 it + k of the chunk: page
    // pi0 + (off0 + k) / page of the staged table, all in 32 bits (a chunk
    // holds at most 2^30 tokens).  A token that is absent (past the length,
    // or its slot outside the cache) reads row 0 of the cache (there is one)
    // and is masked.  Lane (g, r) locates token 16 tile + r.
    auto locate = [&](int it, uint64_t at[2], bool ok[2]) {
      const uint32_t rel0 = (uint32_t)it * kAttIter;
      const uint32_t pi0 = rel0 / (uint32_t)page, off0 = rel0 - pi0 * (uint32_t)page;
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const int k = 16 * tile + r;
        const bool in = (int)rel0 + k < ntok;
        const uint32_t off = off0 + (uint32_t)k;
        const uint32_t qp = small_div(off, (uint32_t)page, inv_page);
        const uint32_t pi = in ? pi0 + qp : 0;
        const uint32_t o = off - qp * (uint32_t)page;
        // (pi is in range either way; the empty asm keeps the compiler from
        // moving the reads under a branch on ok)
        int32_t lim = tlim[pi];
        int64_t base = tbase[pi];
        asm volatile("" : "+v"(lim), "+v"(base));
        ok[tile] = in & ((int32_t)o < lim);
        at[tile] = ok[tile] ? (uint64_t)base + (uint64_t)o * row_bytes : 0;
      }
    };
    auto load_k = [&](const uint64_t at[2], uint4 kx[2][2]) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const uint4* kp = reinterpret_cast<const uint4*>(kbase + at[tile]);
        kx[tile][0] = kp[0];
        kx[tile][1] = kp[1];
      }
    };
    auto load_v = [&](const uint64_t at[2], uint4 vx[2][2]) {
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        const uint4* vp = reinterpret_cast<const uint4*>(vbase + at[tile]);
        vx[tile][0] = vp[0];
        vx[tile][1] = vp[1];
      }
    };
    // Each wave keeps the next iteration's loads in flight behind this
    // one's work: its K loads go out once Q K^T has consumed the current
    // K, its V loads once the current V is in the LDS tile (same registers).
    uint64_t at[2];
    bool ok[2];
    uint4 kx[2][2], vx[2][2];
    if (wave < iters) {
      locate(wave, at, ok);
      load_k(at, kx);
      load_v(at, vx);
    }
    for (int it = wave; it < iters; it += kAttWaves) {
      const bool more = it + kAttWaves < iters;
      uint64_t at_n[2] = {0, 0};
      bool ok_n[2] = {false, false};
      if (more) locate(it + kAttWaves, at_n, ok_n);
      uint64_t okm[2];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) okm[tile] = __ballot(ok[tile]) & 0xFFFF;  // bit j: token 16 tile + j
      // Scores (base 2): lane (g, r) gets tokens 16 tile + 4 g + i of head r.
      float sc[2][4];
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        v4f d = {0.f, 0.f, 0.f, 0.f};
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kx[tile][0].x, kx[tile][0].y),
                                                    __builtin_bit_cast(v8bf, qrow[0]), d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kx[tile][0].z, kx[tile][0].w),
                                                    __builtin_bit_cast(v8bf, qrow[1]), d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kx[tile][1].x, kx[tile][1].y),
                                                    __builtin_bit_cast(v8bf, qrow[2]), d, 0, 0, 0);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(e4m3x8_to_bf16(kx[tile][1].z, kx[tile][1].w),
                                                    __builtin_bit_cast(v8bf, qrow[3]), d, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          sc[tile][i] = ((okm[tile] >> (4 * g + i)) & 1) ? d[i] * cs : -__builtin_inff();
      }
      if (more) load_k(at_n, kx);
      // The V tile to LDS, token-major (read back transposed below; the
      // tile is this wave's own and its LDS operations complete in order).
      // An absent token's weight is 0; its V is zeroed so that whatever row
      // 0 holds cannot turn 0 into NaN.
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        uint4* dst = reinterpret_cast<uint4*>(vt + (16 * tile + r) * kAttVRow + 32 * g);
        dst[0] = ok[tile] ? vx[tile][0] : make_uint4(0, 0, 0, 0);
        dst[1] = ok[tile] ? vx[tile][1] : make_uint4(0, 0, 0, 0);
      }
      if (more) load_v(at_n, vx);
#pragma unroll
      for (int tile = 0; tile < 2; ++tile) {
        at[tile] = at_n[tile];
        ok[tile] = ok_n[tile];
      }
      float mi = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                       fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
      mi = fmaxf(mi, __shfl_xor(mi, 16, 64));
      mi = fmaxf(mi, __shfl_xor(mi, 32, 64));
      const float mn = fmaxf(m, mi);
      // (every token so far skipped: mn = -inf; subtract 0 so that the
      // weights and alpha come out 0 rather than NaN)
      const float mref = (mn == -__builtin_inff() ? 0.f : mn) - kAttWeightExp;
      const float alpha = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      // Weights as fp16 pairs: p = hi + lo to ~2^-21 relative.
      float ps = 0.f;
      _Float16 wh[8], wl[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = __builtin_amdgcn_exp2f(sc[e >> 2][e & 3] - mref);
        ps += pv;
        wh[e] = (_Float16)pv;
        wl[e] = (_Float16)(pv - (float)wh[e]);
      }
      const v8h ph = {wh[0], wh[1], wh[2], wh[3], wh[4], wh[5], wh[6], wh[7]};
      const v8h pl = {wl[0], wl[1], wl[2], wl[3], wl[4], wl[5], wl[6], wl[7]};
      ps += __shfl_xor(ps, 16, 64);
      ps += __shfl_xor(ps, 32, 64);
      // (alpha = 0 on the first tokens: m was -inf; mn = -inf as well gives
      // NaN, where l and the outputs are still 0)
      const float a = mn == -__builtin_inff() ? 1.f : alpha;
      l = l * a + ps;
      if (__ballot(a != 1.f)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] *= a;
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const v2i t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) v2i*)(tr_src + 16 * j));
        const v8h vf = e4m3x8_to_f16((uint32_t)t.x, (uint32_t)t.y);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, ph, acc[j], 0, 0, 0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vf, pl, acc[j], 0, 0, 0);
      }
      asm volatile("" ::: "memory");
    }
  }

  // The 8 waves through LDS (in the V tiles' space, once every wave is
  // past its token loop).
  Part* part = reinterpret_cast<Part*>(vtile);
  __syncthreads();
  if (r < G) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) part[wave][r][16 * j + 4 * g + e] = acc[j][e];
    if (g == 0) {
      part[wave][r][kAttD] = m;
      part[wave][r][kAttD + 1] = l;
    }
  }
  __syncthreads();
  for (int e = tid; e < G * kAttD; e += kAttThreads) {
    const int h = e / kAttD, d = e - h * kAttD;
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kAttWaves; ++w) M = fmaxf(M, part[w][h][kAttD]);
    float L = 0.f, O = 0.f;
    if (M != -__builtin_inff()) {
#pragma unroll
      for (int w = 0; w < kAttWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(part[w][h][kAttD] - M);
        L += part[w][h][kAttD + 1] * f;
        O += part[w][h][d] * f;
      }
    }
    const float v = L > 0.f ? sv * (O / L) : 0.f;
    ob[e] = (uint16_t)f32_to_bf16_rne(v);
  }
}

hipError_t launch_fp8_decode_attention(const uint16_t* q, const float* q_scale,
                                       const uint8_t* k_cache, const uint8_t* v_cache,
                                       const float* k_scale, const float* v_scale,
                                       const int32_t* block_table, const int32_t* seq_lens,
                                       int64_t B, int64_t Hq, int64_t Hkv, int64_t page,
                                       int64_t max_blocks, int64_t num_slots,
                                       float softmax_scale, uint16_t* out, hipStream_t stream) {
  const int G = (int)(Hq / Hkv);
  const dim3 grid((unsigned)(B * Hkv));
#define PRR_ATT(GV)                                                                          \
  case GV:                                                                                   \
    hipLaunchKernelGGL((fp8_decode_attention_kernel<GV>), grid, dim3(kAttThreads), 0, stream, \
                       q, q_scale, k_cache, v_cache, k_scale, v_scale, block_table, seq_lens, \
                       (int)Hq, (int)Hkv, (int)page, (int)max_blocks, num_slots,             \
                       softmax_scale, out);                                                  \
    break;
  switch (G) {
    PRR_ATT(1)
    PRR_ATT(2)
    PRR_ATT(3)
    PRR_ATT(4)
    PRR_ATT(5)
    PRR_ATT(6)
    PRR_ATT(7)
    PRR_ATT(8)
    default:
      return hipErrorInvalidValue;
  }
#undef PRR_ATT
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Split over the tokens of the whole batch (with a caller workspace).  The
// one-pass kernel above gives each (sequence, KV head) its own workgroup, so
// a workgroup reads 128 bytes of every 1 KB cache row (8 KV heads), and
// rows are fetched by 8 workgroups at different times; here one workgroup
// reads whole rows for all KV heads at once, over an equal share of the
// batch's tokens:
//
//  * The batch's cached tokens, sequence after sequence, are cut into
//    gridDim.x equal ranges (one workgroup per CU) of at least
//    kSpanMinTokens tokens (so a sequence meets at most n / 128 + 2
//    workgroups; the ranges past the batch are empty).  Workgroup i walks the
//    sequences its range meets; for each, wave w serves KV head
//    w / (8 / Hkv) over iterations w % (8 / Hkv), ... of the overlap (the
//    same token loop as the one-pass kernel; waves past Hkv (8 / Hkv) idle
//    when Hkv does not divide 8), the waves of a head meet in
//    LDS, and the result (O unnormalized, m, l of every query head) goes to
//    workspace slot i + b: i and b both grow along the batch, so slots are
//    distinct, fewer than gridDim.x + B.
//  * A second kernel combines, per (sequence, query head), the slots of the
//    workgroups whose ranges meet the sequence (for a small batch, four
//    thread groups each take a quarter of them and meet in LDS), and
//    rounds once to bf16.
//
// Workspace: [per, prefix sums of the lengths (B + 1)] as int64, padded to
// 256 bytes, then (gridDim.x + B) x Hq partial results of kAttD + 2 floats.
// ---------------------------------------------------------------------------
constexpr int kSpanMaxB = 2048;         // sequences of one call (prefix sums in LDS)
constexpr int kSpanTablePages = 1024;   // block-table entries staged at a time
constexpr int kSpanPart = kAttD + 2;    // floats of one partial result: O, m, l
constexpr int kSpanMinTokens = 128;     // fewest tokens a workgroup takes (bounds the pieces)
constexpr int kSpanBatch = 8;           // partial results a combining thread loads at once

template <int G>
__global__ __launch_bounds__(kAttThreads) void fp8_decode_attention_span_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ q_scale,
    const uint8_t* __restrict__ k_cache, const uint8_t* __restrict__ v_cache,
    const float* __restrict__ k_scale, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int B, int Hq, int Hkv, int page, int max_blocks,
    int64_t num_slots, float softmax_scale, int64_t* __restrict__ ws_pre,
    float* __restrict__ ws_part) {
  typedef float Part[G][kAttD + 2];
  static_assert(sizeof(Part) * kAttWaves <= kAttWaves * kAttVTile, "partials fit the V tiles");
  __shared__ int64_t pre[kSpanMaxB + 1];             // prefix sums of the clamped lengths
  __shared__ int64_t tbase[kSpanTablePages];
  __shared__ int32_t tlim[kSpanTablePages];
  __shared__ __attribute__((aligned(16))) uint8_t vtile[kAttWaves * kAttVTile];
  __shared__ uint4 qsh[kAttWaves][16 * 4 * 4];        // query operand of each KV head's group
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t n_cap = (int64_t)max_blocks * page;
  auto length = [&](int bb) -> int64_t {
    const int64_t v = seq_lens[bb];
    return min(v < 0 ? (int64_t)0 : v, n_cap);
  };

  // Prefix sums: thread t adds its run of lengths, an inclusive scan of the
  // 512 run totals (two 4 KB buffers in the V tiles' space), then each
  // thread writes the prefixes of its run.
  {
    int64_t* run = reinterpret_cast<int64_t*>(vtile);
    const int per_t = (B + kAttThreads - 1) / kAttThreads;
    const int e0 = min(B, tid * per_t), e1 = min(B, e0 + per_t);
    int64_t tot = 0;
    for (int e = e0; e < e1; ++e) tot += length(e);
    run[tid] = tot;
    __syncthreads();
    int src = 0;
    for (int d = 1; d < kAttThreads; d <<= 1) {
      run[(src ^ kAttThreads) + tid] = run[src + tid] + (tid >= d ? run[src + tid - d] : 0);
      src ^= kAttThreads;
      __syncthreads();
    }
    int64_t at = run[src + tid] - tot;
    for (int e = e0; e < e1; ++e) {
      pre[e] = at;
      at += length(e);
    }
    if (tid == kAttThreads - 1) pre[B] = run[src + tid];
    __syncthreads();
  }
  const int64_t T = pre[B];
  const int64_t per = max((T + gridDim.x - 1) / gridDim.x, (int64_t)kSpanMinTokens);
  if (blockIdx.x == 0) {
    for (int e = tid; e <= B; e += kAttThreads) ws_pre[1 + e] = pre[e];
    if (tid == 0) ws_pre[0] = per;
  }
  const int64_t t0 = (int64_t)blockIdx.x * per, t1 = min(T, t0 + per);
  if (t0 >= t1) return;
  // First sequence that ends past t0 (pre[B] = T > t0, so one exists).
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (pre[mid + 1] > t0) hi = mid;
    else lo = mid + 1;
  }

  // Waves per KV head; waves past Hkv x wpg (Hkv not a divisor of 8) idle.
  const int wpg = kAttWaves / Hkv;
  const int kvh = wave / wpg, sub = wave - kvh * wpg;
  const bool active = kvh < Hkv;
  const int g = lane >> 4, r = lane & 15;
  const uint32_t row_bytes = (uint32_t)Hkv * kAttD;
  const uint8_t* kbase = k_cache + (int64_t)kvh * kAttD + 32 * g;
  const uint8_t* vbase = v_cache + (int64_t)kvh * kAttD + 32 * g;
  uint8_t* vt = vtile + wave * kAttVTile;
  const int tr_tok = 16 * (r >> 3) + 4 * g + ((r >> 1) & 3);
  const uint8_t* tr_src = vt + tr_tok * kAttVRow + 8 * (r & 1);
  const float sq = *q_scale;
  const BlockDiv dq = block_div(sq);
  const float cs = sq * (*k_scale) * softmax_scale * kLog2e;
  const float inv_page = 1.0f / (float)page;
  const uint4* qrow = &qsh[active ? kvh : 0][(r * 4 + g) * 4];
  const int chunk_pages = min(kSpanTablePages, (1 << 30) / page);

  for (int b = lo; b < B && pre[b] < t1; ++b) {
    const int64_t s0 = max(t0, pre[b]) - pre[b], s1 = min(t1, pre[b + 1]) - pre[b];
    if (s1 <= s0) continue;                            // an empty sequence
    __syncthreads();                                   // last segment's readers of qsh / partials
    if (sub == 0 && active) {
      const uint16_t* qh = q + ((int64_t)b * Hq + (int64_t)kvh * G + r) * kAttD + 32 * g;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (r < G) {
          const uint2 c =
              e4m3_chunk_any<true>(*reinterpret_cast<const uint4*>(qh + 8 * j), sq, dq);
          w = __builtin_bit_cast(uint4, e4m3x8_to_bf16(c.x, c.y));
        }
        qsh[kvh][(r * 4 + g) * 4 + j] = w;
      }
    }
    float m = -__builtin_inff(), l = 0.f;
    v4f acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    const int32_t* trow = block_table + (int64_t)b * max_blocks;
    for (int64_t pa = s0 / page; pa * page < s1; pa += chunk_pages) {
      const int64_t c0 = max(s0, pa * page), c1 = min(s1, (pa + chunk_pages) * page);
      const int np = (int)((c1 - 1) / page - pa + 1);
      __syncthreads();                                 // (also publishes qsh on the first pass)
      for (int e = tid; e < np; e += kAttThreads) {
        const int64_t pid = trow[pa + e];
        const int64_t first = pid * page;
        const int64_t lim = pid < 0 ? 0 : min((int64_t)page, max((int64_t)0, num_slots - first));
        tlim[e] = (int32_t)lim;
        tbase[e] = lim > 0 ? first * row_bytes : 0;
      }
      __syncthreads();
      if (active)
        att_chunk<G>(tbase, tlim, (int)(c1 - c0), (uint32_t)(c0 - pa * page), page, inv_page,
                     row_bytes, kbase, vbase, vt, tr_src, qrow, cs, sub, wpg, g, r, m, l, acc);
    }
    // The waves of each KV head through LDS; the segment's partial result
    // of every query head to workspace slot blockIdx.x + b.
    Part* part = reinterpret_cast<Part*>(vtile);
    __syncthreads();
    if (r < G) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) part[wave][r][16 * j + 4 * g + e] = acc[j][e];
      if (g == 0) {
        part[wave][r][kAttD] = m;
        part[wave][r][kAttD + 1] = l;
      }
    }
    __syncthreads();
    float* dst = ws_part + ((int64_t)blockIdx.x + b) * Hq * kSpanPart;
    for (int e = tid; e < Hkv * G * kAttD; e += kAttThreads) {
      const int hh = e / (G * kAttD), rem = e - hh * (G * kAttD);
      const int j = rem / kAttD, d = rem - j * kAttD;
      const int w0 = hh * wpg;
      float M = -__builtin_inff();
      for (int w = 0; w < wpg; ++w) M = fmaxf(M, part[w0 + w][j][kAttD]);
      float L = 0.f, O = 0.f;
      if (M != -__builtin_inff()) {
        for (int w = 0; w < wpg; ++w) {
          const float f = __builtin_amdgcn_exp2f(part[w0 + w][j][kAttD] - M);
          L += part[w0 + w][j][kAttD + 1] * f;
          O += part[w0 + w][j][d] * f;
        }
      }
      float* o = dst + (int64_t)(hh * G + j) * kSpanPart;
      o[d] = O;
      if (d == 0) {
        o[kAttD] = M;
        o[kAttD + 1] = L;
      }
    }
  }
}

// Combines, for sequence b, the partial results of the workgroups whose
// ranges meet it.  A workgroup of 512 threads serves 4 / kGroups query heads
// of one sequence; thread (head, q, d) takes every kGroups-th partial
// result from the q-th on, in one online pass over batches of kSpanBatch
// independent loads, and with kGroups > 1 the groups meet in LDS.  (Many
// partial results per sequence -- a small batch -- take 4 groups; a large
// batch, a few per sequence, takes 1.)
template <int kGroups>
__global__ __launch_bounds__(512) void fp8_decode_attention_combine_kernel(
    const int32_t* __restrict__ seq_lens, int Hq, int64_t n_cap,
    const int64_t* __restrict__ ws_pre, const float* __restrict__ ws_part,
    const float* __restrict__ v_scale, uint16_t* __restrict__ out) {
  constexpr int kHeads = 4 / kGroups;
  __shared__ float gm[4], gl[4], go[4][kAttD];
  const int b = blockIdx.x;
  const int hl = threadIdx.x / (kAttD * kGroups);
  const int q = (threadIdx.x / kAttD) % kGroups, d = threadIdx.x & (kAttD - 1);
  const int h = blockIdx.y * kHeads + hl;
  if (kGroups == 1 && h >= Hq) return;                // (kGroups > 1: one head, h < Hq)
  const int64_t v = seq_lens[b];
  const int64_t n = min(v < 0 ? (int64_t)0 : v, n_cap);
  uint16_t* o = out + ((int64_t)b * Hq + h) * kAttD;
  if (n == 0) {                                       // (uniform in the workgroup)
    if (q == 0) o[d] = 0;
    return;
  }
  const int64_t per = ws_pre[0], P = ws_pre[1 + b];
  const int64_t i0 = P / per, i1 = (P + n - 1) / per;
  const int64_t stride = (int64_t)Hq * kSpanPart;
  const float* base = ws_part + (i0 + b) * stride + (int64_t)h * kSpanPart;
  const int cnt = (int)(i1 - i0 + 1);
  float M = -__builtin_inff(), L = 0.f, O = 0.f;
  for (int k0 = q; k0 < cnt; k0 += kGroups * kSpanBatch) {
    float pm[kSpanBatch], pl[kSpanBatch], po[kSpanBatch];
#pragma unroll
    for (int u = 0; u < kSpanBatch; ++u) {
      const int k = k0 + kGroups * u;
      const bool in = k < cnt;
      const float* pp = base + (in ? (int64_t)k * stride : 0);
      pm[u] = in ? pp[kAttD] : -__builtin_inff();
      pl[u] = pp[kAttD + 1];
      po[u] = pp[d];
    }
    float mb = pm[0];
#pragma unroll
    for (int u = 1; u < kSpanBatch; ++u) mb = fmaxf(mb, pm[u]);
    const float mn = fmaxf(M, mb);
    if (mn == -__builtin_inff()) continue;            // nothing attended so far
    const float a = __builtin_amdgcn_exp2f(M - mn);    // (0 while M is -inf)
    L *= a;
    O *= a;
#pragma unroll
    for (int u = 0; u < kSpanBatch; ++u) {
      const float f = __builtin_amdgcn_exp2f(pm[u] - mn);   // 0 for empty pieces
      L += pl[u] * f;
      O += po[u] * f;
    }
    M = mn;
  }
  if constexpr (kGroups > 1) {
    if (d == 0) {
      gm[q] = M;
      gl[q] = L;
    }
    go[q][d] = O;
    __syncthreads();
    if (q != 0) return;
    float Mt = gm[0];
#pragma unroll
    for (int k = 1; k < kGroups; ++k) Mt = fmaxf(Mt, gm[k]);
    float Lt = 0.f, Ot = 0.f;
    if (Mt != -__builtin_inff()) {
#pragma unroll
      for (int k = 0; k < kGroups; ++k) {
        const float f = __builtin_amdgcn_exp2f(gm[k] - Mt);
        Lt += gl[k] * f;
        Ot += go[k][d] * f;
      }
    }
    L = Lt;
    O = Ot;
  }
  const float res = L > 0.f ? *v_scale * (O / L) : 0.f;
  o[d] = (uint16_t)f32_to_bf16_rne(res);
}

int64_t fp8_decode_attention_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t D) {
  if (D != kAttD || B < 1 || B > kSpanMaxB || Hkv < 1 || Hkv > kAttWaves || Hq < 1 ||
      Hq % Hkv != 0 || Hq / Hkv > 8)
    return 0;
  const int64_t head = ((B + 2) * 8 + 255) / 256 * 256;
  return head + ((int64_t)compute_units() + B) * Hq * kSpanPart * (int64_t)sizeof(float);
}

bool launch_fp8_decode_attention_span(const uint16_t* q, const float* q_scale,
                                      const uint8_t* k_cache, const uint8_t* v_cache,
                                      const float* k_scale, const float* v_scale,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      int64_t B, int64_t Hq, int64_t Hkv, int64_t page,
                                      int64_t max_blocks, int64_t num_slots, float softmax_scale,
                                      uint16_t* out, void* ws, int64_t ws_bytes,
                                      hipStream_t stream, hipError_t* err) {
  const int64_t need = fp8_decode_attention_workspace_bytes(B, Hq, Hkv, kAttD);
  if (need == 0 || ws == nullptr || ws_bytes < need) return false;
  const int G = (int)(Hq / Hkv);
  const int grid = compute_units();
  int64_t* ws_pre = static_cast<int64_t*>(ws);
  float* ws_part = reinterpret_cast<float*>(static_cast<char*>(ws) + ((B + 2) * 8 + 255) / 256 * 256);
#define PRR_ATT_SPAN(GV)                                                                        \
  case GV:                                                                                      \
    hipLaunchKernelGGL((fp8_decode_attention_span_kernel<GV>), dim3(grid), dim3(kAttThreads), 0, \
                       stream, q, q_scale, k_cache, v_cache, k_scale, block_table, seq_lens,    \
                       (int)B, (int)Hq, (int)Hkv, (int)page, (int)max_blocks, num_slots,        \
                       softmax_scale, ws_pre, ws_part);                                         \
    break;
  switch (G) {
    PRR_ATT_SPAN(1)
    PRR_ATT_SPAN(2)
    PRR_ATT_SPAN(3)
    PRR_ATT_SPAN(4)
    PRR_ATT_SPAN(5)
    PRR_ATT_SPAN(6)
    PRR_ATT_SPAN(7)
    PRR_ATT_SPAN(8)
    default:
      *err = hipErrorInvalidValue;
      return true;
  }
#undef PRR_ATT_SPAN
  // about grid / B + 1 partial results per sequence
  if (B * 8 <= grid)
    hipLaunchKernelGGL(fp8_decode_attention_combine_kernel<4>, dim3((unsigned)B, (unsigned)Hq),
                       dim3(512), 0, stream, seq_lens, (int)Hq, max_blocks * page, ws_pre,
                       ws_part, v_scale, out);
  else
    hipLaunchKernelGGL(fp8_decode_attention_combine_kernel<1>,
                       dim3((unsigned)B, (unsigned)((Hq + 3) / 4)), dim3(512), 0, stream,
                       seq_lens, (int)Hq, max_blocks * page, ws_pre, ws_part, v_scale, out);
  *err = hipGetLastError();
  return true;
}


}  // namespace prr

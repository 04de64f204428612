// W8A8 GEMM for many tokens (prefill / log-prob forward): compute-bound, on
// the gfx950 FP8 (or INT8) matrix cores.
//
// A workgroup of 8 waves owns a 256 (m) x TN (n) output tile, TN = 256 or
// 128.  Per 128-deep K block it stages the activation and weight tiles and
// the activation scales of that block in LDS, written there directly by
// buffer loads (no trip through registers), in a two-stage ring: the loads
// for K block kb + 1 are in flight while the waves multiply block kb.  Each
// wave owns a 64 (m) x TN/2 (n) sub-tile, 4 x TN/32 MFMA tiles of 16 x 16,
// whose n range lies in one 128-wide weight block, so its per-block weight
// scale is one scalar.
//
// Block-scaled FP8 (FP8-RL: blockwise W8A8): each 16 x 16 x 128 MFMA covers
// exactly one K block, so it starts from zero and its fp32 result is scaled
// by sa[m, kb] * sw[n / 128, kb] and added to the fp32 accumulator.
// INT8 per channel (FlashRL: INT8 rollout): the int32 accumulator runs over
// the whole K and the two scales are applied once at the end.
//
// LDS rows are 128 bytes; 16-byte chunk c of row r is stored at chunk
// c ^ ((r >> 1) & 7): the 16 rows one fragment read touches then fall on 16
// distinct 16-byte bank groups.
#include <algorithm>

#include "launch.h"
#include "mfma.h"

namespace prr {
namespace {

constexpr int kTileM = 256;
constexpr int kWaves = 8;

// Scales of one K block (FP8): 64 floats per wave slot.  Slots 0..3 hold
// the activation scales of the tile's 256 rows, slot 4 the weight scales of
// its TN / 128 n blocks; slots 5..7 are filled with zeros.
template <int TN>
struct Stage {
  uint8_t a[kTileM * kBlock];   // 32 KB
  uint8_t w[TN * kBlock];       // 32 KB or 16 KB
  float scales[kWaves][64];
};

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100;

constexpr int kWaitVmcnt0 = vmcnt_imm(0);

__device__ __forceinline__ int swz(int r, int c) { return r * kBlock + ((c ^ ((r >> 1) & 7)) << 4); }

// Per-lane byte offsets of the tile loads.  A tile of R rows is loaded as
// R / 8 slabs of 8 rows (1 KB each; lane l fills bytes [16 l, 16 l + 16) of
// a slab), R / 64 consecutive slabs per wave; the chunk a lane fetches
// depends on the slab's parity through the swizzle, hence two offsets.
// Rows past the buffer range (M or N) read zeros.
struct DmaOffsets {
  int even, odd;   // offsets of the wave's first two slab rows at K block 0
};

__device__ __forceinline__ DmaOffsets dma_offsets(int K, int first_row, int lane) {
  const int r0 = first_row + (lane >> 3), r1 = r0 + 8;
  return DmaOffsets{r0 * K + (((lane & 7) ^ ((r0 >> 1) & 7)) << 4),
                    r1 * K + (((lane & 7) ^ ((r1 >> 1) & 7)) << 4)};
}

// Buffer-load instructions one wave issues per stage: 4 activation slabs,
// TN / 64 weight slabs, one scale load (FP8).
template <bool kInt8, int TN>
constexpr int kDmaPerStage = 4 + TN / 64 + (kInt8 ? 0 : 1);

// DMA of K block kb into a stage: both tiles, and (FP8) the activation
// scales (waves 0..3, 64 rows each) and the weight-block scales (wave 4).
// A block at or past kb_end loads nothing (every offset out of range, no
// memory traffic) but still issues the same instructions, so the wait counts
// stay the same.  KB is the row length of the scale arrays.  Branch-free: a branch here makes the register allocator
// shuffle the accumulators around the join.
template <bool kInt8, int TN>
__device__ __forceinline__ void stage_load(Stage<TN>& st, v4i ra, v4i rw, v4i rsa, v4i rsw,
                                           DmaOffsets da, DmaOffsets dw, int K, int KB,
                                           int kb_end, int kb, int wave, int lane) {
  const bool live = kb < kb_end;
  const int soff = live ? kb * kBlock : 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int v = live ? ((q & 1) ? da.odd : da.even) + (q >> 1) * 16 * K : kOutOfRange;
    dma_b128(ra, lds_addr(st.a + (wave * 4 + q) * 1024), v, soff);
  }
  constexpr int kWs = TN / 64;   // weight slabs per wave
#pragma unroll
  for (int q = 0; q < kWs; ++q) {
    const int v = live ? ((q & 1) ? dw.odd : dw.even) + (q >> 1) * 16 * K : kOutOfRange;
    dma_b128(rw, lds_addr(st.w + (wave * kWs + q) * 1024), v, soff);
  }
  if constexpr (!kInt8) {
    const int row = wave < 4 ? wave * 64 + lane : lane;
    const bool valid = live && (wave < 4 || (wave == 4 && lane < TN / kBlock));
    const int vs = valid ? (row * KB + kb) * 4 : kOutOfRange;
    dma_b32(wave < 4 ? rsa : rsw, lds_addr(st.scales[wave]), vs);
  }
}

// Fragment rows always start at a multiple of 16, so the swizzle of row
// base + (lane % 16) depends on the lane only: each lane keeps the byte
// offsets of its two chunks (g and g + 4) within a 16-row group.
struct FragOffsets {
  int lo, hi;
};

__device__ __forceinline__ FragOffsets frag_offsets(int lane) {
  const int r16 = lane & 15, g = lane >> 4;
  return FragOffsets{swz(r16, g), swz(r16, g + 4)};
}

__device__ __forceinline__ v8i lds_frag(const uint8_t* base, int row0, FragOffsets o) {
  const uint8_t* p = base + row0 * kBlock;
  const uint4 lo = *reinterpret_cast<const uint4*>(p + o.lo);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + o.hi);
  return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Accumulators: [weight fragment j][activation fragment i].
template <bool kInt8, int NJ>
struct Acc;
template <int NJ>
struct Acc<false, NJ> {
  v4f v[NJ][4];
};
template <int NJ>
struct Acc<true, NJ> {
  v4i v[NJ][4];
};

// Operand fragments a wave holds when it starts a K block: its 4 activation
// fragments, their per-row scales times the weight-block scale (FP8), and
// its first two weight fragments.
struct Front {
  v8i af[4];
  float s[4];
  v8i wf, wf1;
};

template <bool kInt8, int TN>
__device__ __forceinline__ void load_front(const Stage<TN>& st, Front& f, int wm, int wn, int lane,
                                           FragOffsets o) {
  constexpr int kWaveN = TN / 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.af[i] = lds_frag(st.a, wm * 64 + i * 16, o);
  if constexpr (!kInt8) {
    const float swv = st.scales[4][wn * kWaveN / kBlock];
#pragma unroll
    for (int i = 0; i < 4; ++i) f.s[i] = st.scales[wm][i * 16 + (lane & 15)] * swv;
  }
  f.wf = lds_frag(st.w, wn * kWaveN, o);
  f.wf1 = lds_frag(st.w, wn * kWaveN + 16, o);
}

// FP8 partial products of the previous region, still to be scaled into the
// accumulator, and the scales they take.
struct Pending {
  v4f p[4];
  float s[4];
};

// Region j: 4 MFMAs of weight fragment j against the 4 activation
// fragments.  FP8: each MFMA's product is scaled into the accumulator one
// region later (the FMAs of region j - 1 run here, in the shadow of these
// MFMAs, on results that are complete by now, so they never stall on the
// matrix pipeline); region 0 takes over the last region of the previous
// block.  INT8 accumulates in the MFMA itself.
template <bool kInt8, int NJ>
__device__ __forceinline__ void mma_region(Acc<kInt8, NJ>& acc, int j, const v8i& wf,
                                           const Front& f, Pending& pend) {
  if constexpr (kInt8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc.v[j][i] = mfma_i8x2(wf, f.af[i], acc.v[j][i]);
  } else {
    const int jp = (j + NJ - 1) % NJ;
    v4f p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = mfma_fp8(wf, f.af[i]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc.v[jp][i][r] = fmaf(pend.p[i][r], pend.s[i], acc.v[jp][i][r]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pend.p[i] = p[i];
      pend.s[i] = f.s[i];
    }
  }
}

// One K block.  On entry `cur` holds block kb (landed and published), `f`
// its front fragments (including the first two weight fragments), and block
// kb + 1 is in flight into `nxt`.  Region j reads weight fragment j + 2 and
// runs the 4 MFMAs of fragment j; each region is one scheduling region
// (without the fences the compiler hoists every read and runs out of
// registers).  Region NJ - 3 issues the last read of `cur`; after region
// NJ - 2 the wave waits for its block kb + 1 loads, meets the others at the
// barrier (after which nobody reads `cur`), starts block kb + 2 into `cur`,
// runs the last region and reads the front of block kb + 1 from `nxt`.
// (Reading that front during the last region holds 32 more registers at the
// peak and measured slower; a prefetch distance of one fragment measured
// slower too.)
template <bool kInt8, int TN>
__device__ __forceinline__ void k_block(Stage<TN>& cur, const Stage<TN>& nxt,
                                        Acc<kInt8, TN / 32>& acc, Front& f, Pending& pend, v4i ra,
                                        v4i rw, v4i rsa, v4i rsw, DmaOffsets da, DmaOffsets dw,
                                        int K, int KB, int kb_end, int kb, int wave, int wm,
                                        int wn, int lane,
                                        FragOffsets o) {
  constexpr int NJ = TN / 32, kWaveN = TN / 2;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    v8i w2 = f.wf1;
    if (j + 2 < NJ) w2 = lds_frag(cur.w, wn * kWaveN + (j + 2) * 16, o);
    mma_region<kInt8, NJ>(acc, j, f.wf, f, pend);
    if constexpr (!kInt8) {
      // Issue order: each MFMA followed by 4 of the previous region's scale
      // FMAs (they run while it does), the two LDS reads early.
      if (j + 2 < NJ) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
      if (j + 2 < NJ) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
#pragma unroll
      for (int i = 0; i < 3; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedValu, 4, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (j == NJ - 2) {
      __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);   // this wave's loads of block kb + 1 landed
      lds_barrier();                             // everyone's have; nobody reads `cur` any more
      stage_load<kInt8, TN>(cur, ra, rw, rsa, rsw, da, dw, K, KB, kb_end, kb + 2, wave, lane);
    }
    f.wf = f.wf1;
    f.wf1 = w2;
  }
  load_front<kInt8, TN>(nxt, f, wm, wn, lane, o);
}

// Epilogue staging: the bf16 output tile, rows 0..127 in stage 0 and
// 128..255 in stage 1, 2 TN bytes per row; 16-byte chunk q of row r sits at
// chunk q ^ (r % 16), so the 16 rows one store instruction touches, and the
// chunks one row read touches, fall on distinct banks.
template <int TN>
__device__ __forceinline__ int c_swz(int r, int q) { return r * (2 * TN) + ((q ^ (r & 15)) << 4); }

// Workgroup b -> output tile.  Consecutive workgroups go to the 8 XCDs in
// turn; the remap hands each XCD a contiguous run of logical tiles, and the
// logical order walks groups of 8 m tiles n-tile by n-tile, so the 32
// workgroups an XCD runs at once share 8 activation and 4 weight tiles
// through its L2.
__device__ __forceinline__ void tile_of(int b, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int T = tiles_m * tiles_n;
  const int T8 = T / 8 * 8;
  const int L = b < T8 ? (b % 8) * (T8 / 8) + b / 8 : b;
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = L / per_group;
  const int first_m = group * GM;
  const int gsize = min(GM, tiles_m - first_m);
  const int in_group = L - group * per_group;
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// Output columns [n_base, N) in tiles_m x tiles_n tiles of 256 x TN.
// kPartial: workgroup (b, s) of a grid with gridDim.y = S slices takes K
// blocks [s KB / S, (s + 1) KB / S) of tile b and writes its fp32 partial
// sums (FP8: scaled; INT8: the int32 accumulators, bit-cast) to slab s of
// ws, [S][M][N - n_base], instead of C; a second kernel adds the slabs.
template <bool kInt8, int TN, bool kPartial = false>
__global__ __launch_bounds__(512) void gemm_prefill_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ C, int n_base,
    int tiles_m, int tiles_n, float* __restrict__ ws) {
  constexpr int NJ = TN / 32, kWaveN = TN / 2;
  // Two stages as two objects, so the compiler can tell that the fragment
  // reads of one stage do not wait for the loads into the other.
  __shared__ __align__(16) Stage<TN> st0;
  __shared__ __align__(16) Stage<TN> st1;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 3, wn = wave >> 2;
  int tm, tn;
  tile_of(blockIdx.x, tiles_m, tiles_n, tm, tn);
  const int m0 = tm * kTileM, n0 = n_base + tn * TN;
  const int KB = K / kBlock;
  const int rows_a = min(M - m0, kTileM), rows_w = min(N - n0, TN);
  const int n_slices = kPartial ? (int)gridDim.y : 1, slice = kPartial ? (int)blockIdx.y : 0;
  const int kb_lo = (int)((int64_t)slice * KB / n_slices);
  const int kb_hi = (int)((int64_t)(slice + 1) * KB / n_slices);

  // Every buffer range ends at the tile's last valid row, so rows past M or
  // N (offsets at or beyond it) read zeros.
  const v4i ra = sgpr_rsrc(A + (int64_t)m0 * K, (int64_t)rows_a * K);
  const v4i rw = sgpr_rsrc(W + (int64_t)n0 * K, (int64_t)rows_w * K);
  const v4i rsa = sgpr_rsrc(sa + (int64_t)m0 * KB, (int64_t)rows_a * KB * (int64_t)sizeof(float));
  const int nb0 = n0 / kBlock, NB = (N + kBlock - 1) / kBlock;
  const v4i rsw = sgpr_rsrc(sw + (int64_t)nb0 * KB,
                            (int64_t)min(TN / kBlock, NB - nb0) * KB * (int64_t)sizeof(float));
  const DmaOffsets da = dma_offsets(K, wave * 32, lane);
  const DmaOffsets dw = TN == kTileM ? da : dma_offsets(K, wave * (TN / 8), lane);
  const FragOffsets fo = frag_offsets(lane);
  Acc<kInt8, NJ> acc;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc.v[j][i][r] = 0;

  stage_load<kInt8, TN>(st0, ra, rw, rsa, rsw, da, dw, K, KB, kb_hi, kb_lo, wave, lane);
  stage_load<kInt8, TN>(st1, ra, rw, rsa, rsw, da, dw, K, KB, kb_hi, kb_lo + 1, wave, lane);
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(kDmaPerStage<kInt8, TN>));   // block 0 landed
  lds_barrier();
  Front f;
  load_front<kInt8, TN>(st0, f, wm, wn, lane, fo);
  Pending pend;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pend.p[i] = v4f{0.f, 0.f, 0.f, 0.f};
    pend.s[i] = 0.f;
  }
  // K blocks in pairs (stage 0, stage 1), then an odd last block; one exit
  // keeps the accumulators in place across iterations.
  int kb = kb_lo;
  for (; kb + 2 <= kb_hi; kb += 2) {
    k_block<kInt8, TN>(st0, st1, acc, f, pend, ra, rw, rsa, rsw, da, dw, K, KB, kb_hi, kb, wave,
                       wm, wn, lane, fo);
    k_block<kInt8, TN>(st1, st0, acc, f, pend, ra, rw, rsa, rsw, da, dw, K, KB, kb_hi, kb + 1,
                       wave, wm, wn, lane, fo);
  }
  if (kb < kb_hi)
    k_block<kInt8, TN>(st0, st1, acc, f, pend, ra, rw, rsa, rsw, da, dw, K, KB, kb_hi, kb, wave,
                       wm, wn, lane, fo);
  if constexpr (!kInt8) {   // the last region's products
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        acc.v[NJ - 1][i][r] = fmaf(pend.p[i][r], pend.s[i], acc.v[NJ - 1][i][r]);
  }
  // Every load (the trailing ones are out of range) has landed and every
  // wave is done with the stages before they hold the output tile.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  const int r16 = lane & 15, g = lane >> 4;
  // INT8 epilogue scales: the lane's 4 row scales and 32 channel scales,
  // loaded once, branch-free (clamped indices, zero past M or N), so the
  // epilogue waits for one round trip.  (Loaded per element under bounds
  // branches, they cost one wait per fragment: ~5 us per tile.)
  float sml[4], swl[NJ][4];
  if constexpr (kInt8 && !kPartial) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = (int64_t)m0 + wm * 64 + i * 16 + r16;
      const float x = sa[min(m, (int64_t)M - 1)];
      sml[i] = m < M ? x : 0.f;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = (int64_t)n0 + wn * kWaveN + j * 16 + 4 * g + r;
        const float x = sw[min(n, (int64_t)N - 1)];
        swl[j][r] = n < N ? x : 0.f;
      }
  }
  if constexpr (kPartial) {
    // The partial sums, 16 bytes (4 columns of one row) a lane and
    // fragment, to slab `slice` [M][ncols] of the workspace.
    const int64_t ncols = N - n_base;
    float* slab = ws + (int64_t)slice * M * ncols;
    const bool vec = (ncols & 3) == 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t m = m0 + wm * 64 + i * 16 + r16;
      if (m >= M) continue;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int64_t nl = (int64_t)(n0 - n_base) + wn * kWaveN + j * 16 + 4 * g;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (kInt8) v[r] = __int_as_float(acc.v[j][i][r]);
          else v[r] = acc.v[j][i][r];
        }
        float* dst = slab + m * ncols + nl;
        if (vec && nl + 4 <= ncols) {
          *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (nl + r < ncols) dst[r] = v[r];
        }
      }
    }
    return;
  }
  lds_barrier();

  // Output tile -> bf16 in LDS -> 16-byte row-contiguous stores.
  uint8_t* const lds0 = reinterpret_cast<uint8_t*>(&st0);   // 128 rows of 2 TN bytes
  uint8_t* const lds1 = reinterpret_cast<uint8_t*>(&st1);   // fit in each stage
  uint8_t* half = wm < 2 ? lds0 : lds1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (wm & 1) * 64 + i * 16 + r16;   // row within the half
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int nl = wn * kWaveN + j * 16 + 4 * g;   // column within the tile
      float v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (kInt8) {
          v[r] = (float)acc.v[j][i][r] * (sml[i] * swl[j][r]);
        } else {
          v[r] = acc.v[j][i][r];
        }
      }
      const uint32_t lo = f32_to_bf16_rne(v[0]) | (f32_to_bf16_rne(v[1]) << 16);
      const uint32_t hi = f32_to_bf16_rne(v[2]) | (f32_to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(half + c_swz<TN>(rr, nl >> 3) + ((nl & 4) << 1)) =
          make_uint2(lo, hi);
    }
  }
  lds_barrier();
  const bool vec = (N & 7) == 0;   // rows start 16-byte aligned
  constexpr int kChunks = TN / 8;   // 16-byte chunks per output row
#pragma unroll 4
  for (int it = 0; it < kTileM * kChunks / 512; ++it) {
    const int c = it * 512 + tid;
    const int row = c / kChunks, q = c % kChunks;
    const int64_t m = m0 + row;
    const int64_t n = n0 + q * 8;
    if (m >= M || n >= N) continue;
    const uint8_t* src = (row < 128 ? lds0 : lds1) + c_swz<TN>(row & 127, q);
    const uint4 v = *reinterpret_cast<const uint4*>(src);
    uint16_t* dst = C + m * N + n;
    if (vec && n + 8 <= N) {
      // Streaming store: the output is not read again here, and letting it
      // allocate in L2 evicts the operand tiles other workgroups still read.
      __builtin_nontemporal_store(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w},
                                  reinterpret_cast<v4i*>(dst));
    } else {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 8 && n + e < N; ++e) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
    }
  }
}

// C[:, n_base:] = bf16 of the S partial slabs [S][M][ncols] added in slab
// order (INT8: exactly, then sa[m] sw[n], as the one-pass epilogue does).
// A thread takes 4 consecutive columns of one row (16-byte slab reads when
// ncols % 4 == 0, element by element otherwise).
template <bool kInt8>
__global__ __launch_bounds__(256) void gemm_prefill_tail_reduce_kernel(
    const float* __restrict__ ws, int S, int64_t M, int64_t N, int64_t n_base,
    const float* __restrict__ sa, const float* __restrict__ sw, uint16_t* __restrict__ C) {
  const int64_t ncols = N - n_base, q4 = (ncols + 3) / 4;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= M * q4) return;
  const int64_t m = t / q4, c0 = (t - m * q4) * 4;
  const int64_t MN = M * ncols;
  const float* src = ws + m * ncols + c0;
  float f[4] = {0.f, 0.f, 0.f, 0.f};
  int32_t iacc[4] = {0, 0, 0, 0};
  const bool vec = (ncols & 3) == 0;
  for (int s = 0; s < S; ++s) {
    float v[4];
    if (vec) {
      const float4 x = *reinterpret_cast<const float4*>(src + s * MN);
      v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = c0 + r < ncols ? src[s * MN + r] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr (kInt8) iacc[r] += __float_as_int(v[r]);
      else f[r] += v[r];
    }
  }
  float sm = 1.f, swv[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (kInt8) {
    // the row's scale once, the 4 channel scales in one 16-byte load where
    // they are aligned
    sm = sa[m];
    const int64_t n0 = n_base + c0;
    if (((n0 | N) & 3) == 0 && c0 + 4 <= ncols) {
      const float4 x = *reinterpret_cast<const float4*>(sw + n0);
      swv[0] = x.x; swv[1] = x.y; swv[2] = x.z; swv[3] = x.w;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) swv[r] = c0 + r < ncols ? sw[n0 + r] : 0.f;
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t n = n_base + c0 + r;
    if (c0 + r >= ncols) break;
    float v = f[r];
    if constexpr (kInt8) v = (float)iacc[r] * (sm * swv[r]);
    C[m * N + n] = (uint16_t)f32_to_bf16_rne(v);
  }
}

}  // namespace

// Output columns [n_base, n_end) in 256 x TN tiles.
template <bool kInt8, int TN>
static void launch_cols(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                        int64_t M, int64_t N, int64_t K, uint16_t* C, int64_t n_base,
                        int64_t n_end, hipStream_t stream) {
  const int64_t tiles_m = (M + kTileM - 1) / kTileM, tiles_n = (n_end - n_base + TN - 1) / TN;
  hipLaunchKernelGGL((gemm_prefill_kernel<kInt8, TN>), dim3((unsigned)(tiles_m * tiles_n)),
                     dim3(kWaves * 64), 0, stream, A, sa, W, sw, (int)M, (int)N, (int)K, C,
                     (int)n_base, (int)tiles_m, (int)tiles_n, nullptr);
}

// The shapes the many-token kernel takes (buffer offsets inside one 256-row
// tile are 32-bit; dims fit int), and how its 256-wide tiles fall on the
// compute units: c > 0 trailing tile columns make a last round of at most
// half the units, run apart from the whole rounds before them.
static bool prefill_layout(int64_t M, int64_t N, int64_t K, int64_t* tiles_m, int64_t* tn256,
                           int64_t* c) {
  if (M < 1 || N < 1 || K < kBlock || (int64_t)kTileM * K >= kOutOfRange) return false;
  if (M > 0x7FFFFFFF || N > 0x7FFFFFFF) return false;
  *tiles_m = (M + kTileM - 1) / kTileM;
  if (*tiles_m * ((N + 127) / 128) > 0x7FFFFFFF) return false;
  const int64_t cus = compute_units();
  *tn256 = (N + 255) / 256;
  *c = 0;
  for (int64_t cc = 1; cc < *tn256 && *c == 0; ++cc)
    if (((*tn256 - cc) * *tiles_m) % cus == 0 && 2 * cc * *tiles_m <= cus) *c = cc;
  if (*tiles_m * *tn256 < cus) *c = -1;   // 128-wide tiles throughout
  return true;
}

// With a caller workspace, the trailing tile columns of a long-K layer run
// as 256-wide tiles split over K (S slices, at least 16 K blocks each) on
// the otherwise idle units, their fp32 partial sums added by a second
// kernel, instead of as 128-wide tiles: a 128-wide tile reads its
// activation tile for half the work, and ran at a third of the matrix-core
// busy fraction of the 256-wide ones.  Only for K of 64 blocks or more:
// the slabs (S x M x the tail's columns x 4 bytes, written and read once)
// cost more than they save on short layers.
bool prefill_tail_plan(int64_t M, int64_t N, int64_t K, PrefillTailPlan* plan) {
  int64_t tiles_m, tn256, c;
  if (M <= 128 || !prefill_layout(M, N, K, &tiles_m, &tn256, &c) || c <= 0) return false;
  const int64_t KB = K / kBlock;
  if (KB < 64) return false;
  const int64_t cus = compute_units();
  int64_t S = cus / (c * tiles_m);
  S = std::min<int64_t>(std::min<int64_t>(S, 8), KB / 16);
  if (S < 2) return false;
  plan->n_split = (tn256 - c) * 256;
  plan->S = (int)S;
  plan->bytes = S * M * (N - plan->n_split) * (int64_t)sizeof(float);
  return true;
}

template <bool kInt8>
bool launch_gemm_prefill(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                         int64_t M, int64_t N, int64_t K, uint16_t* C, hipStream_t stream,
                         hipError_t* err) {
  // 256-wide tiles, except that when they leave a last partial round of at
  // most half the compute units busy, the trailing tile columns of that
  // round run as twice as many 128-wide tiles in a second launch (whole
  // rounds first, then one round of half-size tiles instead of a half-empty
  // round of full ones).  With fewer 256-wide tiles than compute units
  // (few tokens), 128-wide tiles throughout.
  int64_t tiles_m, tn256, c;
  if (!prefill_layout(M, N, K, &tiles_m, &tn256, &c)) return false;
  if (c < 0) {
    launch_cols<kInt8, 128>(A, sa, W, sw, M, N, K, C, 0, N, stream);
  } else if (c == 0) {
    launch_cols<kInt8, 256>(A, sa, W, sw, M, N, K, C, 0, N, stream);
  } else {
    const int64_t n_split = (tn256 - c) * 256;
    launch_cols<kInt8, 256>(A, sa, W, sw, M, N, K, C, 0, n_split, stream);
    launch_cols<kInt8, 128>(A, sa, W, sw, M, N, K, C, n_split, N, stream);
  }
  *err = hipGetLastError();
  return true;
}

template <bool kInt8>
bool launch_gemm_prefill_ws(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                            int64_t M, int64_t N, int64_t K, uint16_t* C, float* ws,
                            int64_t ws_bytes, hipStream_t stream, hipError_t* err) {
  PrefillTailPlan pl;
  if (ws == nullptr || !prefill_tail_plan(M, N, K, &pl) || ws_bytes < pl.bytes) return false;
  launch_cols<kInt8, 256>(A, sa, W, sw, M, N, K, C, 0, pl.n_split, stream);
  const int64_t tiles_m = (M + kTileM - 1) / kTileM, tiles_n = (N - pl.n_split + 255) / 256;
  hipLaunchKernelGGL((gemm_prefill_kernel<kInt8, 256, true>),
                     dim3((unsigned)(tiles_m * tiles_n), (unsigned)pl.S), dim3(kWaves * 64), 0,
                     stream, A, sa, W, sw, (int)M, (int)N, (int)K, C, (int)pl.n_split,
                     (int)tiles_m, (int)tiles_n, ws);
  const int64_t threads = M * ((N - pl.n_split + 3) / 4);
  hipLaunchKernelGGL((gemm_prefill_tail_reduce_kernel<kInt8>),
                     dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, stream, ws, pl.S, M,
                     N, pl.n_split, sa, sw, C);
  *err = hipGetLastError();
  return true;
}

template bool launch_gemm_prefill_ws<false>(const uint8_t*, const float*, const uint8_t*,
                                            const float*, int64_t, int64_t, int64_t, uint16_t*,
                                            float*, int64_t, hipStream_t, hipError_t*);
template bool launch_gemm_prefill_ws<true>(const uint8_t*, const float*, const uint8_t*,
                                           const float*, int64_t, int64_t, int64_t, uint16_t*,
                                           float*, int64_t, hipStream_t, hipError_t*);

template bool launch_gemm_prefill<false>(const uint8_t*, const float*, const uint8_t*,
                                         const float*, int64_t, int64_t, int64_t, uint16_t*,
                                         hipStream_t, hipError_t*);
template bool launch_gemm_prefill<true>(const uint8_t*, const float*, const uint8_t*,
                                        const float*, int64_t, int64_t, int64_t, uint16_t*,
                                        hipStream_t, hipError_t*);

}  // namespace prr

// W8A8 GEMM for decode-sized batches (M <= 64 per workgroup; 65-128 rows
// as two row ranges on pairs of workgroups): activation-resident,
// weight-streaming, persistent.
//
// Long-tail decode runs the linear layers at small effective batch, where
// the layer is bound by reading the weight from HBM (TLT notes, section 1:
// the batch shrinks from 128 towards 1 and decode is memory-bound; FlashRL
// article, memory-bound serving speedups).  The weight must therefore be
// read exactly once, at full bandwidth, with nothing else on the path:
//
//  * One 8-wave workgroup per CU loops over 16-channel strips of the
//    output (strip s, s + G, s + 2G, ...; G = grid size), so every CU stays
//    busy to the end with at most one strip of imbalance.
//  * K is split 8 ways across the waves.  Each wave loads the activation
//    fragments of all m-tiles for its K piece once, at the start, and keeps
//    them in registers: activations are never re-read per strip.
//  * The weight reaches each wave through its own ring of R LDS slots.  A
//    slot holds one task, one K block (16 rows x 128 bytes) of one strip,
//    written by two direct-to-LDS buffer loads of 8 whole 128-byte rows
//    (full cache lines, non-temporal: the weight is read once, and the L2
//    is better spent on the activations and the partly written output
//    lines), plus a 4-byte load of the task's weight scale
//    (FP8; INT8: the strip's 16 channel scales, with its first task).  The
//    wave keeps R - 1 tasks in flight: it starts task t + R - 1, waits for
//    task t, reads the fragment from LDS and runs its MFMAs.  No other wave
//    touches the slots, so the ring needs no barrier.  (Loading fragments
//    straight into registers makes each load instruction read 16 rows x 64
//    bytes, half lines, which held the stream near 4.8 TB/s, and the
//    register ring limited how much K a wave could hold.)  Tasks past the
//    end load at out-of-range offsets: no traffic, zeros, no branch.
//  * The 8 partial sums of a strip meet in LDS (two buffers, alternate
//    strips, one barrier per strip); MT waves add them, apply the epilogue
//    and store bf16 while the next strip's first task is in flight.  The
//    barrier orders LDS only, so it does not drain the loads in flight.
//  * Start-up: the ring's first loads, then the activation scales, then
//    the resident activations.  INT8 issues them all before its first
//    wait; FP8 stages its scales in LDS first, which waits for them (and
//    the ring loads ahead of them) before the activations go out (issuing
//    the activations ahead of the staging measured no faster).
//  * Output: a strip writes 32 bytes of each of its M rows.  Strips are
//    mapped to workgroups so that the 4 strips sharing 128-byte output
//    lines run on one XCD, whose L2 merges their writes.  Measured on a
//    64-row problem, the writes still cost about a fifth of the strip time
//    (with no stores at all a strip streams as fast as for one row); staging
//    4 strips in LDS and writing whole lines measured the same.
//
// FP8: per K block, C += sa[m, kb] * sw[n / 128, kb] * MFMA(Wq, Aq) (one
// v_mfma_f32_16x16x128_f8f6f4 per block, zero accumulator).  INT8: the
// int32 MFMA accumulates the wave's whole piece; scales in the epilogue.
#include <algorithm>
#include <atomic>
#include <mutex>

#include "launch.h"
#include "mfma.h"
#include "prr_device.h"

namespace prr {

constexpr int kDecodeWaves = 8;
constexpr int kDecodeThreads = kDecodeWaves * 64;
constexpr int kDecodeRing = 4;       // LDS slots per wave (3 tasks in flight)
constexpr int kLdsBytes = 163840;    // LDS per workgroup on gfx950

// One ring slot: a task's weight block (row r at bytes [128 r, 128 r + 128),
// 16-byte chunk c of the row at position c ^ ((r >> 1) & 7), so the 16 rows
// of one fragment read fall on distinct banks) and its scales.
struct DecodeSlot {
  uint8_t w[16 * kBlock];
  float s[64];
};

// s_waitcnt vmcnt(n) that is also a compiler memory barrier, so no LDS read
// of the awaited slot can be moved above it.
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(n) : "memory");
}

typedef DecodeSlot DecodeRing[kDecodeWaves][kDecodeRing];

// Four fp32 values for P[m, n..n+3], bounds-checked.
__device__ __forceinline__ void store_partial4(float* P, int64_t M, int64_t N, int64_t m,
                                               int64_t n, const float v[4]) {
  if (m >= M) return;
  float* p = P + m * N + n;
  if (n + 3 < N && (N & 3) == 0) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (n + r < N) p[r] = v[r];
  }
}

// The K range of a segment: K/128 blocks starting at block kb_first of
// activation and weight rows that are ld bytes long, whose scale rows hold
// KBs blocks.  A whole layer is {K, 0, K/128}.
struct KSlice {
  int ld, kb_first, KBs;
};

// One segment: the M (<= MT * 16) activation rows at A against the strips
// first, first + step, ... (n_strips of them) of the weight W [N, ld], over
// the K blocks of `ks` (K bytes of each row).  The output rows go to C
// [M, N] as bf16, or, with kPartial, to Pout [M, N] as fp32 partial sums
// (FP8: scaled; INT8: the raw int32 accumulators, bit-cast).  P: K blocks
// of the wave's piece held in registers (>= ceil(K/128 / 8)).  Every wave
// of the workgroup calls it with the same arguments; it starts with a
// barrier (a previous segment's waves may still read the LDS it rewrites)
// and ends with its loads drained.
template <int MT, int P, bool kInt8, bool kPartial = false>
__device__ __forceinline__ void decode_segment(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, int M, int N, int K, KSlice ks, uint16_t* __restrict__ C,
    float* __restrict__ Pout, int first, int step, int n_strips, DecodeRing& ring,
    float* lds_dyn) {
  constexpr int R = kDecodeRing;
  lds_barrier();
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int KB = K / kBlock;
  // This wave's K piece: blocks [kb0, kb0 + pw), pw <= P.
  const int kbase = KB / kDecodeWaves, kextra = KB % kDecodeWaves;
  const int pw = kbase + (wave < kextra ? 1 : 0);
  const int kb0 = wave * kbase + min(wave, kextra);

  const int my_n = __builtin_amdgcn_readfirstlane(n_strips);
  // Strip index math is made provably uniform (readfirstlane) so that the
  // descriptors and LDS addresses live in scalar registers.
  auto strip_n0 = [&](int i) -> int {
    return __builtin_amdgcn_readfirstlane(first + i * step) * 16;
  };

  // Task loads.  Lane l fills bytes [16 l, 16 l + 16) of each half of a
  // slot: row 8 h + l / 8, slot position l % 8, i.e. global chunk
  // (l % 8) ^ ((row >> 1) & 7).
  const int NB = (N + kBlock - 1) / kBlock;
  const int ld = ks.ld, kbf = ks.kb_first;
  const v4i rsw = sgpr_rsrc(sw, kInt8 ? (int64_t)N * 4 : (int64_t)NB * ks.KBs * 4);
  const int lrow0 = lane >> 3, lrow1 = lrow0 + 8;
  const int lofs0 = lrow0 * ld + (((lane & 7) ^ ((lrow0 >> 1) & 7)) << 4);
  const int lofs1 = lrow1 * ld + (((lane & 7) ^ ((lrow1 >> 1) & 7)) << 4);
  auto load_task = [&](int t) {
    const int i = t / P, j = t - i * P;
    const bool live = i < my_n;
    const int n0 = strip_n0(live ? i : 0);
    const int rows = live ? min(16, N - n0) : 0;   // rows past N read zeros
    const v4i rw = sgpr_rsrc(W + (int64_t)n0 * ld, (int64_t)rows * ld);
    const bool jl = j < pw;
    const int kofs = (kbf + kb0 + j) * kBlock;
    DecodeSlot& sl = ring[wave][t % R];
    dma_b128_stream(rw, lds_addr(sl.w), jl ? lofs0 + kofs : kOutOfRange, 0);
    dma_b128_stream(rw, lds_addr(sl.w + 1024), jl ? lofs1 + kofs : kOutOfRange, 0);
    int vs;
    if constexpr (kInt8)
      vs = (live && j == 0 && lane < 16 && n0 + lane < N) ? (n0 + lane) * 4 : kOutOfRange;
    else
      vs = (live && jl && lane == 0) ? ((n0 >> 7) * ks.KBs + kbf + kb0 + j) * 4 : kOutOfRange;
    dma_b32(rsw, lds_addr(sl.s), vs);
  };
  constexpr int kLoadsPerTask = 3;

  // The ring's first R - 1 tasks go out first, then the activation scales
  // and the activations, so that the segment's start-up loads overlap.
#pragma unroll
  for (int q = 0; q < R - 1; ++q) load_task(q);

  // Dynamic LDS: the FP8 activation scales of all rows, transposed to
  // [K block][row] (kept for the whole segment), then two partial-sum
  // exchange buffers used by alternate strips.
  constexpr int kRows = MT * 16;
  float* lsa = lds_dyn;
  float* lred = lds_dyn + (kInt8 ? 0 : kRows * KB);
  constexpr int kRedFloats = kDecodeWaves * MT * 4 * 64;
  float sa_row[MT];
  if constexpr (!kInt8) {
    // kRows x KB <= kRows x 8 P scales: every load is issued before the
    // first store.
    constexpr int kPer = (kRows * 8 * P + kDecodeThreads - 1) / kDecodeThreads;
    float v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * kDecodeThreads;
      const int m = e / KB;
      v[u] = (e < kRows * KB && m < M) ? sa[m * ks.KBs + kbf + (e - m * KB)] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int e = threadIdx.x + u * kDecodeThreads;
      const int m = e / KB, kb = e - m * KB;
      if (e < kRows * KB) lsa[kb * kRows + m] = v[u];
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sa_row[mt] = (mt * 16 + r16 < M) ? sa[mt * 16 + r16] : 0.f;
  }

  // Resident activation fragments of all m-tiles for this wave's K piece.
  // Every CU reads all of the activations (M x K bytes), so how they are
  // fetched matters: a fragment load gives lane 16 g + n 16 bytes of token n,
  // so each group of 16 lanes touches 16 different 64-byte sectors, 16 bytes
  // of each, and at 64 rows fetching the activations that way took 6-8 us of
  // a 36-39 us kernel.  With two or more m-tiles they are instead loaded so
  // that each group of 4 lanes reads one whole 64-byte sector -- instruction
  // h gives lane s chunk 4 h + (s & 3) of token s / 4 -- and one
  // ds_bpermute per register then moves lane 4 n + g to lane 16 g + n: the
  // fragment layout (measured 5-8% faster over the whole GEMM at 32-64
  // rows).  They are issued, block by block, once the FP8 activation scales
  // have been staged in LDS.
  const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(A, (int64_t)M * ld);
  constexpr bool kSectorLoads = MT >= 2;
  v8i afr[MT][P];
#pragma unroll
  for (int j = 0; j < P; ++j)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (kSectorLoads) {
        const int off = (j < pw) ? (mt * 16 + (lane >> 2)) * ld + (kbf + kb0 + j) * kBlock +
                                       (lane & 3) * 16
                                 : kOutOfRange;
        const v4i lo = __builtin_amdgcn_raw_buffer_load_b128(ares, off, 0, 0);
        const v4i hi = __builtin_amdgcn_raw_buffer_load_b128(ares, (j < pw) ? off + 64 : off, 0, 0);
        afr[mt][j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      } else {
        const int m = mt * 16 + r16;
        const int off = (j < pw) ? m * ld + (kbf + kb0 + j) * kBlock + g * 16 : kOutOfRange;
        afr[mt][j] = buffer_load32(ares, off, 0);
      }
    }

  // Wait for the activations here, with nothing queued behind them: an
  // empty asm that consumes the registers makes the compiler place its own
  // wait here rather than at their first use, where it would also wait for
  // the ring loads issued by then.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
      for (int q = 0; q < 8; ++q) asm volatile("" : : "v"(__int_as_float(afr[mt][j][q])));
    if constexpr (kInt8) asm volatile("" : : "v"(sa_row[mt]));
  }
  if constexpr (kSectorLoads) {
    // lane 16 g + n takes lane 4 n + g of the same register (byte address)
    const int src = (((lane & 15) << 2) | (lane >> 4)) << 2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int j = 0; j < P; ++j)
#pragma unroll
        for (int q = 0; q < 8; ++q) afr[mt][j][q] = __builtin_amdgcn_ds_bpermute(src, afr[mt][j][q]);
  }
  if constexpr (!kInt8) lds_barrier();

  // Fragment read offsets of this lane within a slot (chunks g and g + 4).
  const int rbase = r16 * kBlock;
  const int roff_lo = rbase + ((g ^ ((r16 >> 1) & 7)) << 4);
  const int roff_hi = rbase + (((g + 4) ^ ((r16 >> 1) & 7)) << 4);

  // Partial sums of a strip: [wave][mt][lane] x 4 floats, in one of two
  // buffers (strip i uses buffer i & 1).  Waves 0 .. MT-1 add the 8 partial
  // sums of strip i during strip i + 1, right after issuing its first
  // task's loads, so the reduction overlaps that task's memory wait instead
  // of delaying the next load issue.  Buffer i & 1 is written again at the
  // end of strip i + 2, after every wave (the reducers included, having
  // finished) has passed strip i + 1's barrier: one barrier per strip.
  auto red_buf = [&](int i) {
    return reinterpret_cast<float4 (*)[MT][64]>(lred + (i & 1) * kRedFloats);
  };
  float swprev[4] = {0.f, 0.f, 0.f, 0.f};       // INT8: channel scales of the strip being reduced
  auto reduce_strip = [&](int i) {
    if (wave >= MT) return;
    auto red = red_buf(i);
    const int mt = wave;
    const int64_t m = mt * 16 + r16;
    const int64_t n = strip_n0(i) + 4 * g;
    float4 q[kDecodeWaves];
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) q[w] = red[w][mt][lane];
    float v[4];
    if constexpr (kPartial) {
      if constexpr (kInt8) {
        int32_t t[4] = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
          t[0] += __float_as_int(q[w].x);
          t[1] += __float_as_int(q[w].y);
          t[2] += __float_as_int(q[w].z);
          t[3] += __float_as_int(q[w].w);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = __int_as_float(t[r]);
      } else {
        float f[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < kDecodeWaves; ++w) {
          f[0] += q[w].x;
          f[1] += q[w].y;
          f[2] += q[w].z;
          f[3] += q[w].w;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = f[r];
      }
      store_partial4(Pout, M, N, m, n, v);
      return;
    }
    if constexpr (kInt8) {
      int32_t t[4] = {0, 0, 0, 0};
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        t[0] += __float_as_int(q[w].x);
        t[1] += __float_as_int(q[w].y);
        t[2] += __float_as_int(q[w].z);
        t[3] += __float_as_int(q[w].w);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = (float)t[r] * (sa_row[mt] * swprev[r]);
    } else {
      float f[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) {
        f[0] += q[w].x;
        f[1] += q[w].y;
        f[2] += q[w].z;
        f[3] += q[w].w;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) v[r] = f[r];
    }
    store4(C, M, N, m, n, v);
  };

  // FP8: the activation scales of the wave's own K blocks are the same for
  // every strip; held in registers (MT x P of them) they save an LDS read
  // per m-tile and task (1.5% at 64 rows).  Not where the resident
  // activations leave no room: at four m-tiles with more than 4 blocks a
  // wave, the grouped kernel spilled 96 bytes a lane instead of 36.
  constexpr bool kScaleRegs = !kInt8 && (MT < 4 || P <= 4);
  float sareg[MT][P];
  if constexpr (kScaleRegs) {
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        sareg[mt][j] = lsa[min(kb0 + j, KB - 1) * kRows + mt * 16 + r16];
  }
  for (int i = 0; i < my_n; ++i) {
    float accf[MT][4];
    v4i acci[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acci[mt] = v4i{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < 4; ++r) accf[mt][r] = 0.f;
    }
    float swcur[4] = {0.f, 0.f, 0.f, 0.f};
    // An opaque zero keeps the compiler from hoisting the (strip-invariant)
    // activation-scale reads out of the loop into registers.
    int opaque0;
    asm volatile("v_mov_b32 %0, 0" : "=v"(opaque0));
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int t = i * P + j;
      load_task(t + R - 1);
      if (j == 0 && i > 0) reduce_strip(i - 1);
      wait_vmcnt<kLoadsPerTask * (R - 1)>();   // task t has landed
      const DecodeSlot& sl = ring[wave][t % R];
      const uint4 lo = *reinterpret_cast<const uint4*>(sl.w + roff_lo);
      const uint4 hi = *reinterpret_cast<const uint4*>(sl.w + roff_hi);
      const v8i wf = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      if constexpr (kInt8) {
        if (j == 0) {
          // Read now (the slot is reloaded before the reduction needs
          // them): the asm consumes the registers, so the read completes
          // here.
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            swcur[r] = sl.s[4 * g + r];
            asm volatile("" : "+v"(swcur[r]));
          }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acci[mt] = mfma_i8x2(wf, afr[mt][j], acci[mt]);
      } else {
        // (blocks past the piece multiply zeros; their scale index is clamped)
        const int kb = min(kb0 + j, KB - 1);
        const float swv = sl.s[0];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const v4f p = mfma_fp8(wf, afr[mt][j]);
          float sa_v;
          if constexpr (kScaleRegs) sa_v = sareg[mt][j];
          else sa_v = lsa[kb * kRows + mt * 16 + r16 + opaque0];
          const float sc = sa_v * swv;
#pragma unroll
          for (int r = 0; r < 4; ++r) accf[mt][r] = fmaf(p[r], sc, accf[mt][r]);
        }
      }
      // One task per scheduling region: hoisting later tasks' LDS reads, or
      // sinking this task's FMAs to the end of the strip (which keeps every
      // MFMA product live), would cost registers the resident activations
      // need.  The empty volatile asm pins the FMAs before the next task.
      if constexpr (!kInt8) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) asm volatile("" : "+v"(accf[mt][r]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }

    auto red = red_buf(i);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if constexpr (kInt8)
        red[wave][mt][lane] = make_float4(__int_as_float(acci[mt][0]), __int_as_float(acci[mt][1]),
                                          __int_as_float(acci[mt][2]), __int_as_float(acci[mt][3]));
      else
        red[wave][mt][lane] = make_float4(accf[mt][0], accf[mt][1], accf[mt][2], accf[mt][3]);
    }
    if constexpr (kInt8) {
#pragma unroll
      for (int r = 0; r < 4; ++r) swprev[r] = swcur[r];
    }
    lds_barrier();
  }
  if (my_n > 0) reduce_strip(my_n - 1);
  // The trailing (out-of-range) loads land before the LDS is reused.
  wait_vmcnt<0>();
}

// Dense layer: strips l, l + G, l + 2G, ... of one weight (l below).
//
// With m_split = 2 (65 to 128 token rows, more than the registers of one
// workgroup hold) the token rows are cut in two, rows [0, m_half) and
// [m_half, M): workgroups b and b + 8 of every group of 16 take the same
// strips for the two row ranges.  They run on one XCD (workgroup b runs on
// XCD b % 8) at the same time, so the second reads each weight strip from
// that XCD's L2 the first one's loads filled, and the weight streams from
// HBM once.  Every CU fetches only its half of the activations.
template <int MT, int P, bool kInt8>
__global__ __launch_bounds__(512) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ C, int nstrips,
    int m_split, int m_half) {
  __shared__ __align__(16) DecodeRing ring;
  extern __shared__ __align__(16) float lds_dyn[];
  int G = gridDim.x, b = blockIdx.x;
  if (m_split == 2) {
    const int h = (b >> 3) & 1;
    b = (b & 7) | ((b >> 4) << 3);
    G >>= 1;
    const int m0 = h * m_half;
    A += (int64_t)m0 * K;
    sa += kInt8 ? m0 : (int64_t)m0 * (K / kBlock);
    C += (int64_t)m0 * N;
    M = h ? M - m_half : m_half;
  }
  // A strip writes 32 bytes of each output row, a quarter of a 128-byte
  // line.  The strips of a round are mapped so that the 4 strips of each
  // 64-channel line group run on one XCD (workgroup b runs on XCD b % 8),
  // whose L2 then merges the partial line writes: strip l(b) + i G with
  // l = 32 (b / 32) + 4 (b % 8) + (b / 8) % 4, a permutation of [0, G) when
  // G is a multiple of 32.  Counts are uniform; the integer division runs on
  // the vector unit, so the compiler needs telling.
  const int l = (G & 31) == 0 ? (((b >> 5) << 5) | ((b & 7) << 2) | ((b >> 3) & 3)) : b;
  const int my_n = __builtin_amdgcn_readfirstlane((nstrips - l + G - 1) / G);
  decode_segment<MT, P, kInt8>(A, sa, W, sw, M, N, K, KSlice{K, 0, K / kBlock}, C, nullptr, l, G,
                               my_n, ring, lds_dyn);
}

// Split-K decode (a caller-provided workspace): the K blocks are cut into
// S slices; workgroup b works on slice b % S, with its activations for that
// slice resident, over the strips (b / S) + i (G / S), and writes fp32
// partial sums (INT8: int32 accumulators) to workspace slice s [M, N].  A
// second kernel adds the S slices in order and rounds to bf16.  Used where
// one workgroup per strip over all of K would leave CUs idle (few output
// channels) or cannot hold the activations (long K): every CU then reads
// only its slice of the activations, and there are S times more work items.
template <int MT, int P, bool kInt8>
__global__ __launch_bounds__(512) void gemm_decode_splitk_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, int M, int N, int K, int S, int nstrips,
    float* __restrict__ ws) {
  __shared__ __align__(16) DecodeRing ring;
  extern __shared__ __align__(16) float lds_dyn[];
  const int b = blockIdx.x;
  const int s = __builtin_amdgcn_readfirstlane(b % S);
  const int q = __builtin_amdgcn_readfirstlane(b / S);
  const int GQ = (int)gridDim.x / S;
  const int KB = K / kBlock;
  const int kb_first = __builtin_amdgcn_readfirstlane((int)((int64_t)s * KB / S));
  const int kb_end = __builtin_amdgcn_readfirstlane((int)((int64_t)(s + 1) * KB / S));
  const int my_n = __builtin_amdgcn_readfirstlane((nstrips - q + GQ - 1) / GQ);
  decode_segment<MT, P, kInt8, true>(A, sa, W, sw, M, N, (kb_end - kb_first) * kBlock,
                                     KSlice{K, kb_first, KB}, nullptr,
                                     ws + (int64_t)s * M * N, q, GQ, my_n, ring, lds_dyn);
}

// C = bf16(sum over s of ws[s]) in slice order; INT8 adds the int32 slices
// exactly and applies sa[m] sw[n] as the one-pass kernel does.  A thread
// takes 4 consecutive outputs (16-byte reads of every slice when N % 4 ==
// 0, all issued before the adds; element by element otherwise).
constexpr int kReduceSlices = 8;   // slice loads in flight per pass

template <bool kInt8>
__global__ __launch_bounds__(256) void gemm_splitk_reduce_kernel(
    const float* __restrict__ ws, int S, int64_t M, int64_t N, const float* __restrict__ sa,
    const float* __restrict__ sw, uint16_t* __restrict__ C) {
  const int64_t MN = M * N;
  const int64_t i0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i0 >= MN) return;
  float f[4] = {0.f, 0.f, 0.f, 0.f};
  int32_t t[4] = {0, 0, 0, 0};
  if ((N & 3) == 0) {
    for (int k0 = 0; k0 < S; k0 += kReduceSlices) {
      float4 v[kReduceSlices];
#pragma unroll
      for (int u = 0; u < kReduceSlices; ++u)
        v[u] = k0 + u < S ? *reinterpret_cast<const float4*>(ws + (k0 + u) * MN + i0)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int u = 0; u < kReduceSlices; ++u) {
        if (k0 + u >= S) break;
        if constexpr (kInt8) {
          t[0] += __float_as_int(v[u].x);
          t[1] += __float_as_int(v[u].y);
          t[2] += __float_as_int(v[u].z);
          t[3] += __float_as_int(v[u].w);
        } else {
          f[0] += v[u].x;
          f[1] += v[u].y;
          f[2] += v[u].z;
          f[3] += v[u].w;
        }
      }
    }
  } else {
    for (int k = 0; k < S; ++k)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (i0 + r >= MN) break;
        const float x = ws[k * MN + i0 + r];
        if constexpr (kInt8) t[r] += __float_as_int(x); else f[r] += x;
      }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t i = i0 + r;
    if (i >= MN) break;
    float v = f[r];
    if constexpr (kInt8) {
      const int64_t m = i / N, n = i - m * N;
      v = (float)t[r] * (sa[m] * sw[n]);
    }
    C[i] = (uint16_t)f32_to_bf16_rne(v);
  }
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Mixture of experts, FP8 (FP8-RL abstract: the FP8 stack covers MoE
// models).  Rows offsets[e] .. offsets[e+1] - 1 of A go to expert e, whose
// weight is W + e N K with scales sw + e ceil(N/128) K/128.  The work is
// the list of (expert, MT*16-row chunk, 16-channel strip) items of the
// experts that have rows; workgroup b takes a contiguous share of it, so an
// active expert's strips are spread over the workgroups however few experts
// are active, and a workgroup mostly stays on one expert (its activations
// load once per segment).  Offsets are clamped into [0, M]: no access leaves
// the arrays whatever they hold.
//
// Finding the share: the 512 threads read the offsets of 512 experts at a
// time (one load each, all in flight together), and a workgroup prefix sum
// gives each expert's first item in LDS; a binary search there finds the
// first expert of the share.  (Walking the offsets one expert after another
// costs a dependent global load per expert, for every workgroup.)
constexpr int kScanExperts = 512;                 // experts per scan round (= threads)

__device__ __forceinline__ int64_t wave_sum_i64(int64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int MT, int P>
__global__ __launch_bounds__(512) void gemm_grouped_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, const int64_t* __restrict__ offsets, int E, int M, int N, int K,
    uint16_t* __restrict__ C) {
  __shared__ __align__(16) DecodeRing ring;
  __shared__ int64_t first_item[kScanExperts + 1];   // of each expert of the round; [512] = end
  __shared__ int row_lo[kScanExperts], row_hi[kScanExperts];
  __shared__ int64_t wave_part[kDecodeWaves];
  extern __shared__ __align__(16) float lds_dyn[];
  constexpr int kChunk = MT * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int S = (N + 15) / 16;
  const int KB = K / kBlock, NB = (N + kBlock - 1) / kBlock;
  auto rows_of = [&](int e, int64_t& r0, int64_t& r1) {
    r0 = min<int64_t>(max<int64_t>(offsets[e], 0), M);
    r1 = min<int64_t>(max<int64_t>(offsets[e + 1], r0), M);
  };
  auto items_of = [&](int64_t r0, int64_t r1) {
    return (int64_t)S * ((r1 - r0 + kChunk - 1) / kChunk);
  };
  // Total items.
  int64_t mine = 0;
  for (int e = tid; e < E; e += kScanExperts) {
    int64_t r0, r1;
    rows_of(e, r0, r1);
    mine += items_of(r0, r1);
  }
  mine = wave_sum_i64(mine);
  if (lane == 0) wave_part[wave] = mine;
  lds_barrier();
  int64_t total = 0;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) total += wave_part[w];
  total = uniform64(total);
  const int64_t G = gridDim.x;
  const int64_t per = (total + G - 1) / G;
  const int64_t lo = (int64_t)blockIdx.x * per, hi = min(lo + per, total);
  int64_t carry = 0;                                 // items of earlier rounds
  for (int e0 = 0; e0 < E && carry < hi; e0 += kScanExperts) {
    lds_barrier();                                   // wave_part / tables of the last round
    const int cnt = min(kScanExperts, E - e0);
    int64_t r0 = 0, r1 = 0;
    if (tid < cnt) rows_of(e0 + tid, r0, r1);
    const int64_t own = items_of(r0, r1);
    int64_t incl = own;                              // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    if (lane == 63) wave_part[wave] = incl;
    lds_barrier();
    int64_t before = carry;
    for (int w = 0; w < wave; ++w) before += wave_part[w];
    first_item[tid] = before + incl - own;
    row_lo[tid] = (int)r0;
    row_hi[tid] = (int)r1;
    if (tid == kScanExperts - 1) first_item[kScanExperts] = before + incl;
    lds_barrier();
    const int64_t round_end = uniform64(first_item[kScanExperts]);
    if (round_end > lo) {
      // First expert of the round whose items end after lo.
      int a = 0, b = cnt - 1;
      while (a < b) {
        const int mid = (a + b) >> 1;
        if (first_item[mid + 1] > lo) b = mid; else a = mid + 1;
      }
      for (int i = __builtin_amdgcn_readfirstlane(a); i < cnt; ++i) {
        int64_t base = uniform64(first_item[i]);
        if (base >= hi) break;
        const int64_t e_end = uniform64(first_item[i + 1]);
        if (e_end == base) continue;                 // no rows
        const int e = e0 + i;
        const int64_t er0 = __builtin_amdgcn_readfirstlane(row_lo[i]);
        const int64_t er1 = __builtin_amdgcn_readfirstlane(row_hi[i]);
        for (int64_t row0 = er0; row0 < er1 && base < hi; row0 += kChunk, base += S) {
          const int64_t x = max(lo, base), y = min(hi, base + S);
          if (x >= y) continue;
          const int rows = (int)min<int64_t>(kChunk, er1 - row0);
          decode_segment<MT, P, false>(A + row0 * K, sa + row0 * KB, W + (int64_t)e * N * K,
                                       sw + (int64_t)e * NB * KB, rows, N, K, KSlice{K, 0, KB},
                                       C + row0 * N, nullptr, (int)(x - base), 1, (int)(y - x),
                                       ring, lds_dyn);
        }
      }
    }
    carry = round_end;
  }
}

// Scratch for callers that cannot allocate (the split-K partial sums of
// w8a8_block_gemm_scratch).  In host code `scratch` names a host-side
// stand-in, not the device array: its device address comes from
// hipGetSymbolAddress, per device, and only that address is passed to
// kernels.  Every element a split-K call reads is written by the same call
// first, so nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

float* scratch_ptr(hipError_t* err) {
  constexpr int kMaxDevices = 64;
  static std::atomic<void*> addr[kMaxDevices];
  static std::mutex init;
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(init);
    p = addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      // With device `dev` current: its own copy of the array.
      *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (*err != hipSuccess || p == nullptr) {
        if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
        return nullptr;
      }
      addr[dev].store(p, std::memory_order_release);
    }
  }
  return static_cast<float*>(p);
}

// Compute units of the current device (cached per device ordinal).
int compute_units() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int v = 0;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  if (dev < 64) cache[dev].store(v, std::memory_order_relaxed);
  return v;
}

// Smallest P (K blocks per wave) that covers the wave's piece.  Resident
// activations take MT * P * 8 VGPRs.  Every instance compiles without spills
// except MT 4, P 6 (M 33-64, or a half of 65-128 rows, with K 5121-6144),
// which needs 8 (FP8) or 36 (INT8) bytes of scratch per lane: correct, somewhat slower; with a
// workspace those shapes run the split-K kernel only when the layer is
// narrow.  K up to 8192 for M <= 32, 6144 for M <= 64.
template <int MT, bool kInt8>
static bool launch_decode_mt(const uint8_t* A, const float* sa, const uint8_t* W,
                             const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* C,
                             hipStream_t stream, hipError_t* err) {
  const int KB = (int)(K / kBlock);
  const int pw = (KB + kDecodeWaves - 1) / kDecodeWaves;
  const int nstrips = (int)((N + 15) / 16);
  const int cus = compute_units();
  int grid = nstrips < cus ? nstrips : cus;
  // More than 64 rows: two row ranges of at most 64 (the first a multiple of
  // 16, the halves as equal as that allows), on pairs of workgroups; needs
  // a grid of whole groups of 16 and at least one strip per pair.
  const int m_split = M > 64 ? 2 : 1;
  const int m_half = m_split == 2 ? (int)std::min<int64_t>(64, ((M + 1) / 2 + 15) / 16 * 16) : (int)M;
  if (m_split == 2) {
    grid = std::min(cus, 2 * nstrips) / 16 * 16;
    if (grid < 16 || M - m_half > 64) return false;
  }
  const size_t lds = ((size_t)2 * kDecodeWaves * MT * 4 * 64 + (kInt8 ? 0 : (size_t)MT * 16 * KB)) *
                     sizeof(float);
  if (lds + sizeof(DecodeSlot) * kDecodeWaves * kDecodeRing > (size_t)kLdsBytes) return false;
#define PRR_DECODE_P(PV)                                                                  \
  if (pw <= PV) {                                                                         \
    hipLaunchKernelGGL((gemm_decode_kernel<MT, PV, kInt8>), dim3(grid), dim3(512), lds,   \
                       stream, A, sa, W, sw, (int)M, (int)N, (int)K, C, nstrips, m_split,  \
                       m_half);                                                           \
    *err = hipGetLastError();                                                             \
    return true;                                                                          \
  }
  PRR_DECODE_P(2)
  PRR_DECODE_P(3)
  PRR_DECODE_P(4)
  PRR_DECODE_P(5)
  PRR_DECODE_P(6)
  if constexpr (MT <= 2) {
    PRR_DECODE_P(8)
  }
#undef PRR_DECODE_P
  return false;
}

// Split-K plan (one rule for FP8 and INT8, so that the workspace size does
// not depend on the type): for M <= 64, when one pass cannot hold the
// activations (more than 8 Pmax K blocks), or when M > 16 and the layer has
// fewer strips than twice the CUs, cut K into S slices: enough for the register budget, and about 4 work
// items per CU, with at least 8 K blocks per slice.  G workgroups, a multiple
// of S; the workspace is S x M x N fp32.
bool splitk_plan(int64_t M, int64_t N, int64_t K, SplitPlan* plan) {
  if (M < 1 || M > 64 || N < 1 || K < kBlock || K % kBlock != 0) return false;
  if (128 * K >= 0x7FFFFF00LL || N > 0x1FFFFFF0LL || 64 * K >= 0x7FFFFF00LL) return false;
  const int64_t KB = K / kBlock;
  if (4 * ((N + kBlock - 1) / kBlock) * KB >= 0x7FFFFF00LL) return false;
  const int mt = (int)((M + 15) / 16);
  const int MT = mt <= 2 ? mt : 4;
  const int64_t pmax = MT <= 2 ? 8 : 6;
  const int64_t nstrips = (N + 15) / 16;
  const int cus = compute_units();
  const bool one_pass = (KB + kDecodeWaves - 1) / kDecodeWaves <= pmax;
  // (At M <= 16 the one-pass kernel's start-up is short, and the second
  // launch of the split costs more than the idle CUs on narrow layers.)
  if (one_pass && (nstrips >= 2 * cus || M <= 16)) return false;
  const int64_t s_regs = (KB + kDecodeWaves * pmax - 1) / (kDecodeWaves * pmax);
  const int64_t s_bal = (4 * cus + nstrips - 1) / nstrips;
  int64_t S = std::max(s_regs, s_bal);
  S = std::min<int64_t>(S, std::min<int64_t>(KB / kDecodeWaves, 32));
  if (S < 2 || S < s_regs) return false;
  const int64_t kbs = (KB + S - 1) / S;                 // longest slice
  const size_t lds = ((size_t)2 * kDecodeWaves * MT * 4 * 64 + (size_t)MT * 16 * kbs) * sizeof(float);
  if (lds + sizeof(DecodeSlot) * kDecodeWaves * kDecodeRing > (size_t)kLdsBytes) return false;
  if (M * N * S > (int64_t)1 << 40) return false;
  plan->S = (int)S;
  plan->G = std::max<int>((int)S, cus / (int)S * (int)S);
  plan->MT = MT;
  plan->pw = (int)((kbs + kDecodeWaves - 1) / kDecodeWaves);
  plan->bytes = M * N * S * (int64_t)sizeof(float);
  return true;
}

template <int MT, bool kInt8>
static bool launch_splitk_mt(const uint8_t* A, const float* sa, const uint8_t* W,
                             const float* sw, int64_t M, int64_t N, int64_t K, float* ws,
                             const SplitPlan& pl, uint16_t* C, hipStream_t stream,
                             hipError_t* err) {
  const int KB = (int)(K / kBlock);
  const int kbs = (KB + pl.S - 1) / pl.S;
  const int nstrips = (int)((N + 15) / 16);
  const size_t lds = ((size_t)2 * kDecodeWaves * MT * 4 * 64 + (kInt8 ? 0 : (size_t)MT * 16 * kbs)) *
                     sizeof(float);
  bool launched = false;
#define PRR_SPLIT_P(PV)                                                                         if (!launched && pl.pw <= PV) {                                                                 hipLaunchKernelGGL((gemm_decode_splitk_kernel<MT, PV, kInt8>), dim3(pl.G), dim3(512), lds,                        stream, A, sa, W, sw, (int)M, (int)N, (int)K, pl.S, nstrips, ws);           launched = true;                                                                            }
  PRR_SPLIT_P(2)
  PRR_SPLIT_P(3)
  PRR_SPLIT_P(4)
  PRR_SPLIT_P(5)
  PRR_SPLIT_P(6)
  if constexpr (MT <= 2) {
    PRR_SPLIT_P(8)
  }
#undef PRR_SPLIT_P
  if (!launched) return false;
  const int64_t MN = M * N;
  hipLaunchKernelGGL((gemm_splitk_reduce_kernel<kInt8>), dim3((unsigned)((MN + 1023) / 1024)),
                     dim3(256), 0, stream, ws, pl.S, M, N, sa, sw, C);
  *err = hipGetLastError();
  return true;
}

template <bool kInt8>
bool launch_gemm_decode_splitk(const uint8_t* A, const float* sa, const uint8_t* W,
                               const float* sw, int64_t M, int64_t N, int64_t K, float* ws,
                               int64_t ws_bytes, uint16_t* C, hipStream_t stream,
                               hipError_t* err) {
  SplitPlan pl;
  if (ws == nullptr || !splitk_plan(M, N, K, &pl) || ws_bytes < pl.bytes) return false;
  switch (pl.MT) {
    case 1: return launch_splitk_mt<1, kInt8>(A, sa, W, sw, M, N, K, ws, pl, C, stream, err);
    case 2: return launch_splitk_mt<2, kInt8>(A, sa, W, sw, M, N, K, ws, pl, C, stream, err);
    case 4: return launch_splitk_mt<4, kInt8>(A, sa, W, sw, M, N, K, ws, pl, C, stream, err);
    default: return false;
  }
}

template bool launch_gemm_decode_splitk<false>(const uint8_t*, const float*, const uint8_t*,
                                               const float*, int64_t, int64_t, int64_t, float*,
                                               int64_t, uint16_t*, hipStream_t, hipError_t*);
template bool launch_gemm_decode_splitk<true>(const uint8_t*, const float*, const uint8_t*,
                                              const float*, int64_t, int64_t, int64_t, float*,
                                              int64_t, uint16_t*, hipStream_t, hipError_t*);

template <bool kInt8>
bool launch_gemm_decode(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                        int64_t M, int64_t N, int64_t K, uint16_t* C, hipStream_t stream,
                        hipError_t* err) {
  // 32-bit offsets: a 16-row strip and all of A must stay below 2^31 bytes.
  // Activations of more than 64 rows do not fit in one workgroup's
  // registers: 65-128 rows take two row ranges on pairs of workgroups.
  // Scale offsets (4 N for INT8, 4 ceil(N/128) K/128 for FP8) are 32-bit too.
  if (M < 1 || M > 128 || K < kBlock || 128 * K >= 0x7FFFFF00LL || N > 0x1FFFFFF0LL) return false;
  if (M * K >= 0x7FFFFF00LL) return false;
  if (!kInt8 && 4 * ((N + kBlock - 1) / kBlock) * (K / kBlock) >= 0x7FFFFF00LL) return false;
  if (!kInt8 && (std::min<int64_t>(64, (M + 15) / 16 * 16)) * (K / kBlock) > 8192) return false;
  if (M > 64) return launch_decode_mt<4, kInt8>(A, sa, W, sw, M, N, K, C, stream, err);
  switch ((M + 15) / 16) {
    case 1: return launch_decode_mt<1, kInt8>(A, sa, W, sw, M, N, K, C, stream, err);
    case 2: return launch_decode_mt<2, kInt8>(A, sa, W, sw, M, N, K, C, stream, err);
    case 3:
    case 4: return launch_decode_mt<4, kInt8>(A, sa, W, sw, M, N, K, C, stream, err);
    default: return false;
  }
}

// As launch_decode_mt; the MT 4 instances with P 5 and 6 (more than 32 rows
// for some expert, K 4097-6144) spill 36 and 208 bytes per lane.
template <int MT>
static bool launch_grouped_mt(const uint8_t* A, const float* sa, const uint8_t* W,
                              const float* sw, const int64_t* offsets, int64_t E, int64_t M,
                              int64_t N, int64_t K, uint16_t* C, hipStream_t stream,
                              hipError_t* err) {
  const int KB = (int)(K / kBlock);
  const int pw = (KB + kDecodeWaves - 1) / kDecodeWaves;
  const size_t lds = ((size_t)2 * kDecodeWaves * MT * 4 * 64 + (size_t)MT * 16 * KB) * sizeof(float);
  const size_t tables = (kScanExperts + 1) * 8 + kScanExperts * 8 + kDecodeWaves * 8;
  if (lds + tables + sizeof(DecodeSlot) * kDecodeWaves * kDecodeRing > (size_t)kLdsBytes)
    return false;
  const int grid = compute_units();
#define PRR_GROUPED_P(PV)                                                                  \
  if (pw <= PV) {                                                                          \
    hipLaunchKernelGGL((gemm_grouped_kernel<MT, PV>), dim3(grid), dim3(512), lds, stream, A, \
                       sa, W, sw, offsets, (int)E, (int)M, (int)N, (int)K, C);             \
    *err = hipGetLastError();                                                              \
    return true;                                                                           \
  }
  PRR_GROUPED_P(2)
  PRR_GROUPED_P(3)
  PRR_GROUPED_P(4)
  PRR_GROUPED_P(5)
  PRR_GROUPED_P(6)
  if constexpr (MT <= 2) {
    PRR_GROUPED_P(8)
  }
#undef PRR_GROUPED_P
  return false;
}

bool launch_gemm_grouped(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                         const int64_t* offsets, int64_t E, int64_t M, int64_t N, int64_t K,
                         int64_t rows_hint, uint16_t* C, hipStream_t stream, hipError_t* err) {
  // Same 32-bit offset limits as the dense kernel (per expert weight).
  if (K < kBlock || 128 * K >= 0x7FFFFF00LL || N > 0x1FFFFFF0LL) return false;
  if (4 * ((N + kBlock - 1) / kBlock) * (K / kBlock) >= 0x7FFFFF00LL) return false;
  if (64 * K >= 0x7FFFFF00LL) return false;
  if (rows_hint <= 16) return launch_grouped_mt<1>(A, sa, W, sw, offsets, E, M, N, K, C, stream, err);
  if (rows_hint <= 32) return launch_grouped_mt<2>(A, sa, W, sw, offsets, E, M, N, K, C, stream, err);
  return launch_grouped_mt<4>(A, sa, W, sw, offsets, E, M, N, K, C, stream, err);
}

template bool launch_gemm_decode<false>(const uint8_t*, const float*, const uint8_t*, const float*,
                                        int64_t, int64_t, int64_t, uint16_t*, hipStream_t,
                                        hipError_t*);
template bool launch_gemm_decode<true>(const uint8_t*, const float*, const uint8_t*, const float*,
                                       int64_t, int64_t, int64_t, uint16_t*, hipStream_t,
                                       hipError_t*);

}  // namespace prr

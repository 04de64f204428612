// W8A8 GEMM for decode-sized batches (M <= 64): activation-resident,
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
//    fragments of all m-tiles for its K piece (and their FP8 scales) once,
//    at the start, and keeps them in registers: activations are never
//    re-read per strip.
//  * Per strip a wave loads only the weight fragments of its K piece
//    (16 rows x 32 bytes per lane per K block, through raw buffer loads)
//    into a D-deep register ring, so D strips are in flight; the ring is
//    branch-free (pieces or strips past the end load at an out-of-range
//    offset: no traffic, zeros) so the compiler waits only for the oldest
//    stage.
//  * The 8 partial sums of a strip meet in LDS; MT waves add them, apply
//    the epilogue and store bf16.  The barriers order LDS only, so they do
//    not drain the weight loads in flight.
//
// FP8: per K block, C += sa[m, kb] * sw[n / 128, kb] * MFMA(Wq, Aq) (one
// v_mfma_f32_16x16x128_f8f6f4 per block, zero accumulator).  INT8: the
// int32 MFMA accumulates the wave's whole piece; scales in the epilogue.
#include <atomic>

#include "launch.h"
#include "mfma.h"
#include "prr_device.h"

namespace prr {

constexpr int kDecodeWaves = 8;

// D: strips of weight fragments held per wave.  Each fragment is reloaded
// (for strip i + D) right after the MFMA that consumed it, so about D
// strips are always in flight.
template <int MT, int P, int D, bool kInt8>
__global__ __launch_bounds__(512) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ sa, const uint8_t* __restrict__ W,
    const float* __restrict__ sw, int M, int N, int K, uint16_t* __restrict__ C, int nstrips) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, g = lane >> 4;
  const int KB = K / kBlock;
  // This wave's K piece: blocks [kb0, kb0 + pw), pw <= P.
  const int kbase = KB / kDecodeWaves, kextra = KB % kDecodeWaves;
  const int pw = kbase + (wave < kextra ? 1 : 0);
  const int kb0 = wave * kbase + min(wave, kextra);

  // Resident activation fragments of all m-tiles for this wave's K piece.
  const __amdgpu_buffer_rsrc_t ares = buffer_rsrc(A, (int64_t)M * K);
  v8i afr[MT][P];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int m = mt * 16 + r16;
      const int off = (j < pw) ? m * K + (kb0 + j) * kBlock + g * 16 : kOutOfRange;
      afr[mt][j] = buffer_load32(ares, off, 0);
    }

  // LDS: the FP8 activation scales of all rows, transposed to [K block][row]
  // (kept for the whole kernel), then the partial-sum exchange buffer.
  extern __shared__ float lds_dyn[];
  constexpr int kRows = MT * 16;
  float* lsa = lds_dyn;
  float* lred = lds_dyn + (kInt8 ? 0 : kRows * KB);
  if constexpr (!kInt8) {
    for (int e = threadIdx.x; e < kRows * KB; e += blockDim.x) {
      const int m = e / KB, kb = e - m * KB;
      lsa[kb * kRows + m] = (m < M) ? sa[(int64_t)m * KB + kb] : 0.f;
    }
    lds_barrier();
  }

  const int G = gridDim.x;
  const int my_n = (nstrips - (int)blockIdx.x + G - 1) / G;   // strips of this workgroup

  // Strip index math is made provably uniform (readfirstlane) so that the
  // weight resource and the scale addresses live in scalar registers: a
  // vector load of a scale would queue behind every weight refill in flight.
  auto strip_n0 = [&](int i) -> int64_t {
    return (int64_t)__builtin_amdgcn_readfirstlane((int)blockIdx.x + i * G) * 16;
  };

  // INT8 epilogue scales: the lane's token rows (once) and, per strip, the
  // lane's four channels (loaded with the strip's weight, D strips ahead).
  float sa_row[MT];
  float4 swq[D];
  const __amdgpu_buffer_rsrc_t swres = buffer_rsrc(sw, kInt8 ? (int64_t)N * 4 : 0);
  if constexpr (kInt8) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) sa_row[mt] = (mt * 16 + r16 < M) ? sa[mt * 16 + r16] : 0.f;
  }
  auto load_swq = [&](int i) -> float4 {
    const int off = (i < my_n) ? (int)(strip_n0(i) + 4 * g) * 4 : kOutOfRange;
    const v4i v = __builtin_amdgcn_raw_buffer_load_b128(swres, off, 0, 0);
    return make_float4(__int_as_float(v[0]), __int_as_float(v[1]), __int_as_float(v[2]),
                       __int_as_float(v[3]));
  };

  // Weight ring: D strips, each this wave's P fragments of one strip.
  v8i wbuf[D][P];
  auto load_strip = [&](int d, int i) {
    const bool live = i < my_n;                                 // workgroup-uniform
    const int64_t n0 = strip_n0(i);
    const int64_t rows = live ? min<int64_t>(16, N - n0) : 0;
    const __amdgpu_buffer_rsrc_t wres = buffer_rsrc(W + (live ? n0 : 0) * K, rows * K);
#pragma unroll
    for (int j = 0; j < P; ++j) {
      const int off = (j < pw) ? r16 * K + (kb0 + j) * kBlock + g * 16 : kOutOfRange;
      wbuf[d][j] = buffer_load32(wres, off, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < D; ++d) {
    load_strip(d, d);
    if constexpr (kInt8) swq[d] = load_swq(d);
    __builtin_amdgcn_sched_barrier(0);
  }

  auto red = reinterpret_cast<float (*)[MT][4][64]>(lred);      // [wave][mt][r][lane]

  for (int t = 0; t < my_n; t += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = t + d;
      const int64_t n0 = strip_n0(i);
      float accf[MT][4];
      v4i acci[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        acci[mt] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 4; ++r) accf[mt][r] = 0.f;
      }
      // The next strip's fragments for this slot, issued one by one as the
      // current ones are consumed (same resource for the whole strip).
      const int inext = i + D;
      const bool nlive = inext < my_n;
      const int64_t nn0 = strip_n0(inext);
      const int64_t nrows = nlive ? min<int64_t>(16, N - nn0) : 0;
      const __amdgpu_buffer_rsrc_t nres = buffer_rsrc(W + (nlive ? nn0 : 0) * K, nrows * K);
      float4 swcur = make_float4(0.f, 0.f, 0.f, 0.f);
      if constexpr (kInt8) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acci[mt] = mfma_i8x2(wbuf[d][j], afr[mt][j], acci[mt]);
          wbuf[d][j] = buffer_load32(
              nres, (j < pw) ? r16 * K + (kb0 + j) * kBlock + g * 16 : kOutOfRange, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        swcur = swq[d];
        swq[d] = load_swq(inext);
        __builtin_amdgcn_sched_barrier(0);
      } else {
        // The strip's weight scales for this wave's K blocks (the index is
        // clamped into the array; blocks past the piece multiply zeros).
        const float* swrow =
            sw + (int64_t)__builtin_amdgcn_readfirstlane((int)(((i < my_n ? n0 : 0) >> 7) * KB));
        // An opaque zero keeps the compiler from hoisting the (strip-
        // invariant) activation-scale reads out of the loop into registers.
        int opaque0;
        asm volatile("v_mov_b32 %0, 0" : "=v"(opaque0));
#pragma unroll
        for (int j = 0; j < P; ++j) {
          const int kb = min(kb0 + j, KB - 1);
          const float swv = swrow[kb];
          // (blocks past the piece read a real scale and multiply zeros)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) {
            const v4f p = mfma_fp8(wbuf[d][j], afr[mt][j]);
            const float sc = lsa[kb * kRows + mt * 16 + r16 + opaque0] * swv;
#pragma unroll
            for (int r = 0; r < 4; ++r) accf[mt][r] = fmaf(p[r], sc, accf[mt][r]);
          }
          wbuf[d][j] = buffer_load32(
              nres, (j < pw) ? r16 * K + (kb0 + j) * kBlock + g * 16 : kOutOfRange, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      // Add the 8 partial sums of the strip through LDS (for 8 m-tiles the
      // upper 4 waves first fold theirs into the lower 4, so the buffer
      // holds at most 4 waves x 8 KB).
      constexpr int kHeld = (MT > 4) ? kDecodeWaves / 2 : kDecodeWaves;
      if constexpr (MT > 4) {
        if (wave >= kHeld) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              red[wave - kHeld][mt][r][lane] =
                  kInt8 ? __int_as_float(acci[mt][r]) : accf[mt][r];
        }
        lds_barrier();
        if (wave < kHeld) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              if constexpr (kInt8) acci[mt][r] += __float_as_int(red[wave][mt][r][lane]);
              else accf[mt][r] += red[wave][mt][r][lane];
            }
        }
        lds_barrier();
      }
      if (wave < kHeld) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[wave][mt][r][lane] = kInt8 ? __int_as_float(acci[mt][r]) : accf[mt][r];
      }
      lds_barrier();
      if (i < my_n && wave < MT) {
        const int mt = wave;
        const int64_t m = mt * 16 + r16;
        const int64_t n = n0 + 4 * g;
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (kInt8) {
            int32_t tsum = 0;
#pragma unroll
            for (int w = 0; w < kHeld; ++w) tsum += __float_as_int(red[w][mt][r][lane]);
            const float sn = r == 0 ? swcur.x : r == 1 ? swcur.y : r == 2 ? swcur.z : swcur.w;
            v[r] = (float)tsum * (sa_row[mt] * sn);
          } else {
            float fsum = 0.f;
#pragma unroll
            for (int w = 0; w < kHeld; ++w) fsum += red[w][mt][r][lane];
            v[r] = fsum;
          }
        }
        store4(C, M, N, m, n, v);
      }
      lds_barrier();
    }
  }
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

// Largest P (K blocks per wave) whose resident activations fit the
// register budget for each m-tile count: MT * P * 8 VGPRs.
template <int MT, bool kInt8>
static bool launch_decode_mt(const uint8_t* A, const float* sa, const uint8_t* W,
                             const float* sw, int64_t M, int64_t N, int64_t K, uint16_t* C,
                             hipStream_t stream, hipError_t* err) {
  const int KB = (int)(K / kBlock);
  const int pw = (KB + kDecodeWaves - 1) / kDecodeWaves;
  const int nstrips = (int)((N + 15) / 16);
  const int cus = compute_units();
  const int grid = nstrips < cus ? nstrips : cus;
  const size_t lds =
      ((size_t)(MT > 4 ? kDecodeWaves / 2 : kDecodeWaves) * MT * 4 * 64 + (kInt8 ? 0 : (size_t)MT * 16 * KB)) *
      sizeof(float);
  constexpr int D = MT >= 4 ? 1 : 2;
#define PRR_DECODE_P(PV)                                                                  \
  if (pw <= PV) {                                                                         \
    hipLaunchKernelGGL((gemm_decode_kernel<MT, PV, D, kInt8>), dim3(grid), dim3(512), lds, \
                       stream, A, sa, W, sw, (int)M, (int)N, (int)K, C, nstrips);         \
    *err = hipGetLastError();                                                             \
    return true;                                                                          \
  }
  // Resident activations take MT * P * 8 of a wave's 256 registers and the
  // weight ring D * P * 8; these ranges compile without spills (so K up to
  // 6144 for M <= 16, 5120 for M <= 32, 4096 for M <= 64).
  PRR_DECODE_P(2)
  PRR_DECODE_P(3)
  PRR_DECODE_P(4)
  if constexpr (MT <= 2) {
    PRR_DECODE_P(5)
  }
  if constexpr (MT <= 1) {
    PRR_DECODE_P(6)
  }
#undef PRR_DECODE_P
  return false;
}

template <bool kInt8>
bool launch_gemm_decode(const uint8_t* A, const float* sa, const uint8_t* W, const float* sw,
                        int64_t M, int64_t N, int64_t K, uint16_t* C, hipStream_t stream,
                        hipError_t* err) {
  // 32-bit offsets: a 16-row strip and all of A must stay below 2^31 bytes.
  // Activations of more than 64 rows do not fit in registers.
  if (M < 1 || M > 64 || K < kBlock || 128 * K >= 0x7FFFFF00LL || N > 0x7FFFFFFFLL - 16)
    return false;
  if (!kInt8 && ((M + 15) / 16 * 16) * (K / kBlock) > 8192) return false;   // scales in LDS
  switch ((M + 15) / 16) {
    case 1: return launch_decode_mt<1, kInt8>(A, sa, W, sw, M, N, K, C, stream, err);
    case 2: return launch_decode_mt<2, kInt8>(A, sa, W, sw, M, N, K, C, stream, err);
    case 3:
    case 4: return launch_decode_mt<4, kInt8>(A, sa, W, sw, M, N, K, C, stream, err);
    default: return false;
  }
}

template bool launch_gemm_decode<false>(const uint8_t*, const float*, const uint8_t*, const float*,
                                        int64_t, int64_t, int64_t, uint16_t*, hipStream_t,
                                        hipError_t*);
template bool launch_gemm_decode<true>(const uint8_t*, const float*, const uint8_t*, const float*,
                                       int64_t, int64_t, int64_t, uint16_t*, hipStream_t,
                                       hipError_t*);

}  // namespace prr

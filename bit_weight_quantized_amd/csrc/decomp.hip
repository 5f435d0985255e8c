// Multi-Scale Dequant activation decomposition ("Multi-Scale Dequant:
// Eliminating Dequantization Bottleneck via Activation Decomposition for
// Efficient LLM Inference", Abstract): fp16 activations are split into int8
// slices with per-token scales, so that x ~= sum_j s_j[m] * A_j[m, k].
//
// Per token m, in fp64 with r = x: s_j = fp32(max_k |r| / 127);
// A_j = clamp(rint(r / s_j), -127, 127); r <- r - s_j * A_j (the product and
// the difference are exact for up to three slices, so contraction cannot
// change the result).  The residuals and maxima are exact fp64 values; each
// rint is decided from an fp32 estimate, with an exact fp64 sign test where
// the estimate is near a half-integer (decide127), which gives the same
// integers as the fp64 division.
//
// The slices are written in the byte order the int8 matrix-core product reads
// them in (the operand layout below); the plain [slice][token][K] layout is
// written as well when the caller asks for it.
//
// Operand layout of a token row: per 64 K positions, 64 bytes; K position
// 64 b + 32 h + 8 kb + e is stored at byte 64 b + 16 kb + 8 h + p(e) with
// p(0..7) = 0, 2, 4, 6, 1, 3, 5, 7 -- so lane kb's 16-byte A operand of a
// 16x16x64 product is contiguous and its bytes pair with the weight bytes
// the masks (w & 0x0F0F0F0F), ((w >> 4) & 0x0F0F0F0F) produce from the stored
// nibble order (codes c0 c4 c1 c5 | c2 c6 c3 c7 of each 8).
#include "w4_device.h"
#include "w4_internal.h"

#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int kDecompThreads = 256;
// few rows (M <= kFewRows): one 1024-thread workgroup per row, so that the
// grid still fills the CUs and each thread walks a quarter of the row
constexpr int kDecompWide = 1024;
constexpr int kFewRows = 512;

template <int T>
__device__ __forceinline__ double block_max(double v, double* red) {
  v = wave_max_d(v);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < T / kWave; ++w) r = fmax(r, red[w]);
  return r;
}

__device__ __forceinline__ int code_byte(const uint32_t (&w)[2], int i) {
  return (int)(int8_t)(uint8_t)(w[i / 4] >> (8 * (i % 4)));
}

__device__ __forceinline__ uint32_t pack4(int a0, int a1, int a2, int a3) {
  return (uint32_t)(a0 & 0xFF) | ((uint32_t)(a1 & 0xFF) << 8) | ((uint32_t)(a2 & 0xFF) << 16) |
         ((uint32_t)(a3 & 0xFF) << 24);
}

// One workgroup per token row, passes over the (cache-resident) row: the
// absmax, then one pass per slice.  Pass j rebuilds the residual from x and
// the earlier slices' codes (kept in registers when the row is; decided again,
// identically, when it is re-read) and gathers the next residual's absmax
// (adaptive scales).  With FIXED (two slices), the second slice uses the first
// slice's step divided by 254: A_2 = clamp(rint((254 r_1) / s_1)), and its
// reported scale is fp32(s_1 / 254).  Each thread takes 8 consecutive
// elements per step (one 16-byte load) and stores them as one 8-byte piece of
// the operand layout (and of the plain layout if asked).
constexpr double kFixedRatio = 254.0;

// T threads per workgroup.  CH > 0: the row's K <= CH * 8 * (row threads)
// positions are read once into registers (CH 16-byte chunks per thread) and
// every pass reuses them; CH = 0 re-reads the row in each pass.  WR: one wave
// per row (K <= 512, T / 64 rows per workgroup, wave-level maxima);
// otherwise the workgroup takes one row.
template <int NS, bool FIXED, int CH, bool WR, int T>
__global__ __launch_bounds__(T) void decompose_kernel(
    const uint16_t* __restrict__ x, int M, int K, int8_t* __restrict__ slices_op, int8_t* __restrict__ slices_out,
    float* __restrict__ tok_scale) {
  static_assert(!FIXED || NS == 2, "the fixed ratio defines a second slice");
  static_assert(!WR || CH == 1, "a wave's row is one chunk per lane");
  __shared__ double red[T / kWave];
  constexpr int kRowThreads = WR ? kWave : T;
  constexpr int kStep = 8 * kRowThreads;
  const int rt = WR ? (int)threadIdx.x % kWave : (int)threadIdx.x;  // thread within the row
  const int m = WR ? (int)blockIdx.x * (T / kWave) + (int)threadIdx.x / kWave : (int)blockIdx.x;
  if (WR && m >= M) return;  // whole waves leave; no workgroup barrier follows in this variant
  const uint16_t* xr = x + (size_t)m * K;
  auto row_max = [&](double v) {  // the WR variant has no workgroup barrier
    if constexpr (WR) return wave_max_d(v);
    else return block_max<T>(v, red);
  };

  u32x4 xc[CH > 0 ? CH : 1];
  if constexpr (CH > 0) {
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int k = 8 * rt + c * kStep;
      if (k < K) xc[c] = *reinterpret_cast<const u32x4*>(xr + k);
    }
  }
  // f(c, k, w) for each of this thread's 16-byte chunks w (K positions k ..
  // k + 7; c its register slot when the row is cached, else 0)
  auto for_chunks = [&](auto&& f) {
    if constexpr (CH > 0) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int k = 8 * rt + c * kStep;
        if (k < K) f(c, k, xc[c]);
      }
    } else {
      for (int k = 8 * rt; k < K; k += kStep) f(0, k, *reinterpret_cast<const u32x4*>(xr + k));
    }
  };
  auto load8 = [&](const u32x4& w, double* v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)half_bits_to_float((uint16_t)(w[i] & 0xFFFFu));
      v[2 * i + 1] = (double)half_bits_to_float((uint16_t)(w[i] >> 16));
    }
  };
  // K positions k .. k + 7 of slice j: plain and operand layouts
  auto store8 = [&](int j, int k, const int (&a)[8]) {
    const size_t row = ((size_t)j * M + m) * K;
    if (slices_out)
      *reinterpret_cast<u32x2*>(slices_out + row + k) = u32x2{pack4(a[0], a[1], a[2], a[3]), pack4(a[4], a[5], a[6], a[7])};
    const int kk = k % 64, h = kk / 32, kb = (kk % 32) / 8;
    *reinterpret_cast<u32x2*>(slices_op + row + (k - kk) + 16 * kb + 8 * h) =
        u32x2{pack4(a[0], a[4], a[1], a[5]), pack4(a[2], a[6], a[3], a[7])};
  };

  double amax = 0.0;
  for_chunks([&](int, int, const u32x4& w) {
    double v[8];
    load8(w, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmax(amax, fabs(v[i]));
  });
  amax = row_max(amax);
  double s[NS];
  float inv[NS];
  s[0] = (double)(float)(amax / 127.0);
  inv[0] = s[0] != 0.0 ? (float)(1.0 / s[0]) : 0.f;
  // the earlier slices' codes of the cached chunks (plain order), so a pass
  // rebuilds its residual without deciding those codes again
  uint32_t codes[NS > 1 ? NS - 1 : 1][CH > 0 ? CH : 1][2];

#pragma unroll
  for (int j = 0; j < NS; ++j) {
    double amax_next = 0.0;
    for_chunks([&](int c, int k, const u32x4& w) {
      double v[8];
      load8(w, v);
      int a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        double r = v[i];
#pragma unroll
        for (int jj = 0; jj < j; ++jj) {  // earlier slices' residual (exact in fp64)
          const double qq = CH > 0 ? (double)code_byte(codes[jj][c], i) : (double)decide127(r, s[jj], inv[jj]);
          r = r - s[jj] * qq;
        }
        float q;
        if (FIXED && j == 1)
          q = decide127(kFixedRatio * r, s[0], inv[0]);
        else
          q = decide127(r, s[j], inv[j]);
        a[i] = (int)q;
        if (!FIXED && j + 1 < NS) amax_next = fmax(amax_next, fabs(r - s[j] * (double)q));
      }
      store8(j, k, a);
      if constexpr (CH > 0) {
        if (j + 1 < NS) {
          codes[j][c][0] = pack4(a[0], a[1], a[2], a[3]);
          codes[j][c][1] = pack4(a[4], a[5], a[6], a[7]);
        }
      }
    });
    if (FIXED && j == 1) {
      if (rt == 0) tok_scale[(size_t)M + m] = (float)(s[0] / kFixedRatio);
    } else {
      if (rt == 0) tok_scale[(size_t)j * M + m] = (float)s[j];
      if (!FIXED && j + 1 < NS) {
        s[j + 1] = (double)(float)(row_max(amax_next) / 127.0);
        inv[j + 1] = s[j + 1] != 0.0 ? (float)(1.0 / s[j + 1]) : 0.f;
      }
    }
  }
}

// The largest of a block's non-negative values given as bits whose unsigned
// order is the values' order (fp16 or fp32 magnitudes): within each DPP row
// of 16 lanes (pairs, quads, half-mirror, mirror; the moves fold into the
// integer maximum), over the wave's four rows (lane reads), then over the
// waves through LDS.
template <int T>
__device__ __forceinline__ uint32_t block_max_bits(uint32_t v, uint32_t* red) {
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true));
  v = max(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true));
  const uint32_t w = max(max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16)),
                         max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48)));
  __syncthreads();  // the previous maximum's reads of red are done
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = w;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int i = 1; i < T / kWave; ++i) r = max(r, red[i]);
  return r;
}

// Lean variant for one or two slices with the row cached in registers (K <=
// 32 T): the same decisions as decompose_kernel, with fewer instructions.
//  * The absmax comes from the magnitude bits (an integer maximum: the bit
//    pattern of |x| orders like the value for finite x).
//  * r_1 = x - s_1 A_1 is one fp32 fma, and exact: for A_1 = 0 it is x;
//    otherwise |x| >= s_1 / 2, so x is a multiple of s_1's ulp (the fp16 grid
//    at |x| is at least 2^12 of them) and |r_1| <= s_1 / 2 is at most 2^23 of
//    them.  So the residual maximum is an fp32 maximum, and the second slice
//    decides from r_1 (adaptive: rint(r_1 / s_2); fixed ratio:
//    rint(fl32(254 r_1) / s_1), the estimate the product with the
//    decomposition in its K loop uses, within 2^-15 of the quotient).
//  * Each 16-byte chunk's 8 decisions take their fast fp32 form, and the exact
//    decide127 runs for all 8 only when one of them lies within 2^-14 of a
//    half-integer (about 1 chunk in 1000): one branch per chunk, not one per
//    decision.
//  * fp64 remains for the scales and inside those fallbacks.
template <int NS, bool FIXED, int T>
__global__ __launch_bounds__(T) void decompose_lean_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                           int8_t* __restrict__ slices_op,
                                                           int8_t* __restrict__ slices_out,
                                                           float* __restrict__ tok_scale) {
  static_assert(NS == 1 || NS == 2, "one or two slices");
  static_assert(!FIXED || NS == 2, "the fixed ratio defines a second slice");
  constexpr int CH = 4;
  constexpr int kStep = 8 * T;
  __shared__ uint32_t red[T / kWave];
  const int rt = (int)threadIdx.x;
  const int m = (int)blockIdx.x;
  const uint16_t* xr = x + (size_t)m * K;

  u32x4 xc[CH];
  uint32_t mag = 0;  // two 15-bit magnitudes per word: the larger of each half
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = 8 * rt + c * kStep;
    xc[c] = k < K ? *reinterpret_cast<const u32x4*>(xr + k) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w = xc[c][i] & 0x7FFF7FFFu;
      mag = max(mag, max(w & 0xFFFFu, w >> 16));
    }
  }
  const double amax = (double)half_bits_to_float((uint16_t)block_max_bits<T>(mag, red));
  const double s1 = (double)(float)(amax / 127.0);
  const float inv1 = s1 != 0.0 ? (float)(1.0 / s1) : 0.f;
  const float s1f = (float)s1;

  auto store8 = [&](int j, int k, const int (&a)[8]) {
    const size_t row = ((size_t)j * M + m) * K;
    if (slices_out)
      *reinterpret_cast<u32x2*>(slices_out + row + k) = u32x2{pack4(a[0], a[1], a[2], a[3]), pack4(a[4], a[5], a[6], a[7])};
    const int kk = k % 64, h = kk / 32, kb = (kk % 32) / 8;
    *reinterpret_cast<u32x2*>(slices_op + row + (k - kk) + 16 * kb + 8 * h) =
        u32x2{pack4(a[0], a[4], a[1], a[5]), pack4(a[2], a[6], a[3], a[7])};
  };
  float rf[NS > 1 ? CH : 1][8];  // r_1 = x - s_1 A_1 (exact)
  uint32_t mag2 = 0;             // bits of max |r_1|
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = 8 * rt + c * kStep;
    if (k >= K) continue;
    float xf[8], q[8];
    float dmax = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xf[2 * i] = half_bits_to_float((uint16_t)(xc[c][i] & 0xFFFFu));
      xf[2 * i + 1] = half_bits_to_float((uint16_t)(xc[c][i] >> 16));
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) q[i] = rint127_fast(xf[i], inv1, dmax);
    if (near127(dmax)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = decide127((double)xf[i], s1, inv1);
    }
    int a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (int)q[i];  // in [-127, 127]: |x / s_1| <= 127.0001
    store8(0, k, a);
    if constexpr (NS > 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rf[c][i] = fmaf(-s1f, q[i], xf[i]);
        mag2 = max(mag2, __float_as_uint(fabsf(rf[c][i])));
      }
    }
  }
  if (rt == 0) tok_scale[m] = (float)s1;
  if constexpr (NS == 1) return;

  double s2 = s1;
  float inv2 = inv1;
  if constexpr (!FIXED) {
    s2 = (double)(float)((double)__uint_as_float(block_max_bits<T>(mag2, red)) / 127.0);
    inv2 = s2 != 0.0 ? (float)(1.0 / s2) : 0.f;
  }
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = 8 * rt + c * kStep;
    if (k >= K) continue;
    float q[8];
    float dmax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float n = FIXED ? (float)kFixedRatio * rf[c][i] : rf[c][i];
      q[i] = rint127_fast(n, inv2, dmax);
    }
    if (near127(dmax)) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double r = (double)rf[c][i];
        q[i] = FIXED ? decide127(kFixedRatio * r, s1, inv1) : decide127(r, s2, inv2);
      }
    }
    int a[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = (int)q[i];  // |r_1 / s_2|, |254 r_1 / s_1| <= 127.0001
    store8(1, k, a);
  }
  if (rt == 0) tok_scale[(size_t)M + m] = FIXED ? (float)(s1 / kFixedRatio) : (float)s2;
}

}  // namespace

int launch_decompose(const uint16_t* x, int M, int K, int nslices, bool fixed, int8_t* slices_op, int8_t* slices_out,
                     float* tok_scale, hipStream_t s) {
// rows cached in registers: the lean kernel for one or two slices
#define W4_DECOMP_CACHED(NS, FX, T)                                                                                 \
  do {                                                                                                             \
    if constexpr (NS <= 2)                                                                                         \
      hipLaunchKernelGGL((decompose_lean_kernel<NS, FX, T>), dim3(M), dim3(T), 0, s, x, M, K, slices_op, slices_out, \
                         tok_scale);                                                                               \
    else                                                                                                           \
      hipLaunchKernelGGL((decompose_kernel<NS, FX, 4, false, T>), dim3(M), dim3(T), 0, s, x, M, K, slices_op,       \
                         slices_out, tok_scale);                                                                   \
  } while (0)
#define W4_DECOMP(NS, FX)                                                                                        \
  do {                                                                                                          \
    constexpr int kRows = kDecompThreads / kWave;                                                               \
    if (K <= 8 * kWave)                                                                                         \
      hipLaunchKernelGGL((decompose_kernel<NS, FX, 1, true, kDecompThreads>), dim3((M + kRows - 1) / kRows),    \
                         dim3(kDecompThreads), 0, s, x, M, K, slices_op, slices_out, tok_scale);                \
    else if (M <= kFewRows && K <= 4 * 8 * kDecompWide)                                                         \
      W4_DECOMP_CACHED(NS, FX, kDecompWide);                                                                    \
    else if (K <= 4 * 8 * kDecompThreads)                                                                       \
      W4_DECOMP_CACHED(NS, FX, kDecompThreads);                                                                 \
    else                                                                                                        \
      hipLaunchKernelGGL((decompose_kernel<NS, FX, 0, false, kDecompThreads>), dim3(M), dim3(kDecompThreads), 0, \
                         s, x, M, K, slices_op, slices_out, tok_scale);                                         \
  } while (0)
  if (fixed)
    W4_DECOMP(2, true);
  else if (nslices == 1)
    W4_DECOMP(1, false);
  else if (nslices == 2)
    W4_DECOMP(2, false);
  else
    W4_DECOMP(3, false);
#undef W4_DECOMP
#undef W4_DECOMP_CACHED
  return check_launch("decompose");
}

}  // namespace w4

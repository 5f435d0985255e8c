// Multi-Scale Dequant activation decomposition ("Multi-Scale Dequant:
// Eliminating Dequantization Bottleneck via Activation Decomposition for
// Efficient LLM Inference", Abstract): fp16 activations are split into int8
// slices with per-token scales, so that x ~= sum_j s_j[m] * A_j[m, k].
//
// Per token m, in fp64 with r = x: s_j = fp32(max_k |r| / 127);
// A_j = clamp(rint(r / s_j), -127, 127); r <- r - s_j * A_j (the product and
// the difference are exact for up to three slices, so contraction cannot
// change the result).  All decisions are IEEE fp64 operations, bit-identical
// to any other correct fp64 evaluation.
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

__device__ __forceinline__ double quant127(double r, double s) {
  return s != 0.0 ? fmin(fmax(rint(r / s), -127.0), 127.0) : 0.0;
}

__device__ __forceinline__ uint32_t pack4(int a0, int a1, int a2, int a3) {
  return (uint32_t)(a0 & 0xFF) | ((uint32_t)(a1 & 0xFF) << 8) | ((uint32_t)(a2 & 0xFF) << 16) |
         ((uint32_t)(a3 & 0xFF) << 24);
}

// One workgroup per token row, passes over the (cache-resident) row: the
// absmax, then one pass per slice.  Pass j recomputes the residual from x and
// the earlier slices exactly as before and gathers the next residual's absmax
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
  // f(k, w) for each of this thread's 16-byte chunks w (K positions k .. k + 7)
  auto for_chunks = [&](auto&& f) {
    if constexpr (CH > 0) {
#pragma unroll
      for (int c = 0; c < CH; ++c) {
        const int k = 8 * rt + c * kStep;
        if (k < K) f(k, xc[c]);
      }
    } else {
      for (int k = 8 * rt; k < K; k += kStep) f(k, *reinterpret_cast<const u32x4*>(xr + k));
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
  for_chunks([&](int, const u32x4& w) {
    double v[8];
    load8(w, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmax(amax, fabs(v[i]));
  });
  amax = row_max(amax);
  double s[NS];
  s[0] = (double)(float)(amax / 127.0);

#pragma unroll
  for (int j = 0; j < NS; ++j) {
    double amax_next = 0.0;
    for_chunks([&](int k, const u32x4& w) {
      double v[8];
      load8(w, v);
      int a[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        double r = v[i];
#pragma unroll
        for (int jj = 0; jj < j; ++jj) r = r - s[jj] * quant127(r, s[jj]);  // earlier slices' residual
        double q;
        if (FIXED && j == 1)
          q = s[0] != 0.0 ? fmin(fmax(rint((kFixedRatio * r) / s[0]), -127.0), 127.0) : 0.0;
        else
          q = quant127(r, s[j]);
        a[i] = (int)q;
        if (!FIXED && j + 1 < NS) amax_next = fmax(amax_next, fabs(r - s[j] * q));
      }
      store8(j, k, a);
    });
    if (FIXED && j == 1) {
      if (rt == 0) tok_scale[(size_t)M + m] = (float)(s[0] / kFixedRatio);
    } else {
      if (rt == 0) tok_scale[(size_t)j * M + m] = (float)s[j];
      if (!FIXED && j + 1 < NS) s[j + 1] = (double)(float)(row_max(amax_next) / 127.0);
    }
  }
}

}  // namespace

int launch_decompose(const uint16_t* x, int M, int K, int nslices, bool fixed, int8_t* slices_op, int8_t* slices_out,
                     float* tok_scale, hipStream_t s) {
#define W4_DECOMP(NS, FX)                                                                                        \
  do {                                                                                                          \
    constexpr int kRows = kDecompThreads / kWave;                                                               \
    if (K <= 8 * kWave)                                                                                         \
      hipLaunchKernelGGL((decompose_kernel<NS, FX, 1, true, kDecompThreads>), dim3((M + kRows - 1) / kRows),    \
                         dim3(kDecompThreads), 0, s, x, M, K, slices_op, slices_out, tok_scale);                \
    else if (M <= kFewRows && K <= 4 * 8 * kDecompWide)                                                         \
      hipLaunchKernelGGL((decompose_kernel<NS, FX, 4, false, kDecompWide>), dim3(M), dim3(kDecompWide), 0, s, x, \
                         M, K, slices_op, slices_out, tok_scale);                                               \
    else if (K <= 4 * 8 * kDecompThreads)                                                                       \
      hipLaunchKernelGGL((decompose_kernel<NS, FX, 4, false, kDecompThreads>), dim3(M), dim3(kDecompThreads), 0, \
                         s, x, M, K, slices_op, slices_out, tok_scale);                                         \
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
  return check_launch("decompose");
}

}  // namespace w4

// Multi-Scale Dequant activation decomposition ("Multi-Scale Dequant:
// Eliminating Dequantization Bottleneck via Activation Decomposition for
// Efficient LLM Inference", Abstract): fp16 activations are split into int8
// slices with per-token scales, so that x ~= sum_j s_j[m] * A_j[m, k].
//
// Per token m, in fp64 with r = x: s_j = fp32(max_k |r| / 127);
// A_j = clamp(rint(r / s_j), -127, 127); r <- r - s_j * A_j (the product is
// exact, so contraction cannot change the result).  All decisions are IEEE
// fp64 operations, bit-identical to any other correct fp64 evaluation.
//
// Besides the slices and scales, the kernel emits the per-group slice sums
// SA_j[m, g] = sum_{k in g} A_j[m, k] (exact int32), which the integer product
// kernel needs to apply each group's zero point after accumulation.
#include "w4_device.h"
#include "w4_internal.h"

#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int kDecompThreads = 256;
constexpr int kDecompMaxGroups = 512;  // K / G per row held in LDS

__device__ __forceinline__ double block_max(double v, double* red) {
  v = wave_max_d(v);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double r = red[0];
  for (int w = 1; w < kDecompThreads / kWave; ++w) r = fmax(r, red[w]);
  return r;
}

__device__ __forceinline__ double quant127(double r, double s) {
  return s != 0.0 ? fmin(fmax(rint(r / s), -127.0), 127.0) : 0.0;
}

// Sum over the `seg` consecutive lanes (a power of two) that share one group.
__device__ __forceinline__ int segment_sum(int v, int seg) {
  for (int off = 1; off < seg; off <<= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ uint32_t pack4(int a0, int a1, int a2, int a3) {
  return (uint32_t)(a0 & 0xFF) | ((uint32_t)(a1 & 0xFF) << 8) | ((uint32_t)(a2 & 0xFF) << 16) |
         ((uint32_t)(a3 & 0xFF) << 24);
}

// One workgroup per token row, passes over the (cache-resident) row: the
// absmax, then slice 1 (with the residual's absmax), then slice 2, whose
// residual is recomputed from x and slice 1 exactly as before.  Each thread
// takes 8 consecutive elements per step (one 16-byte load); the G / 8 lanes
// that share a group add their slice sums with register shuffles, and one of
// them adds the result into the row's LDS group total.
template <int NS>
__global__ __launch_bounds__(kDecompThreads) void decompose_kernel(
    const uint16_t* __restrict__ x, int M, int K, int G, int8_t* __restrict__ slices,
    float* __restrict__ tok_scale, int32_t* __restrict__ gsum) {
  __shared__ double red[kDecompThreads / kWave];
  __shared__ int gs[NS][kDecompMaxGroups];
  constexpr int kStep = 8 * kDecompThreads;
  const int m = blockIdx.x;
  const int ng = K / G;
  const int seg = G / 8;
  const int lane = threadIdx.x % kWave;
  const uint16_t* xr = x + (size_t)m * K;
  for (int t = threadIdx.x; t < NS * ng; t += kDecompThreads) gs[t / ng][t % ng] = 0;

  auto load8 = [&](int k, double* v) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(xr + k);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = (double)half_bits_to_float((uint16_t)(w[i] & 0xFFFFu));
      v[2 * i + 1] = (double)half_bits_to_float((uint16_t)(w[i] >> 16));
    }
  };

  double amax = 0.0;
  for (int k = 8 * threadIdx.x; k < K; k += kStep) {
    double v[8];
    load8(k, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmax(amax, fabs(v[i]));
  }
  amax = block_max(amax, red);  // also orders the gs clearing before the adds below
  const double s1 = (double)(float)(amax / 127.0);

  double amax2 = 0.0;
  for (int k = 8 * threadIdx.x; k < K; k += kStep) {
    double v[8];
    load8(k, v);
    int a[8], sum = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double q = quant127(v[i], s1);
      a[i] = (int)q;
      sum += a[i];
      amax2 = fmax(amax2, fabs(v[i] - s1 * q));
    }
    *reinterpret_cast<u32x2*>(slices + (size_t)m * K + k) = u32x2{pack4(a[0], a[1], a[2], a[3]),
                                                                   pack4(a[4], a[5], a[6], a[7])};
    sum = segment_sum(sum, seg);  // whole segments are active together (K % G == 0)
    if (lane % seg == 0) atomicAdd(&gs[0][k / G], sum);
  }
  if (threadIdx.x == 0) tok_scale[m] = (float)s1;
  if constexpr (NS == 2) {
    amax2 = block_max(amax2, red);
    const double s2 = (double)(float)(amax2 / 127.0);
    for (int k = 8 * threadIdx.x; k < K; k += kStep) {
      double v[8];
      load8(k, v);
      int a[8], sum = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const double r1 = v[i] - s1 * quant127(v[i], s1);
        a[i] = (int)quant127(r1, s2);
        sum += a[i];
      }
      *reinterpret_cast<u32x2*>(slices + ((size_t)M + m) * K + k) =
          u32x2{pack4(a[0], a[1], a[2], a[3]), pack4(a[4], a[5], a[6], a[7])};
      sum = segment_sum(sum, seg);
      if (lane % seg == 0) atomicAdd(&gs[1][k / G], sum);
    }
    if (threadIdx.x == 0) tok_scale[(size_t)M + m] = (float)s2;
  }
  __syncthreads();
  for (int t = threadIdx.x; t < NS * ng; t += kDecompThreads) {
    const int j = t / ng, g = t - j * ng;
    gsum[((size_t)j * M + m) * ng + g] = gs[j][g];
  }
}

}  // namespace

int launch_decompose(const uint16_t* x, int M, int K, int G, int nslices, int8_t* slices,
                     float* tok_scale, int32_t* gsum, hipStream_t s) {
  if (K / G > kDecompMaxGroups)
    return fail(-2, "w4_gemm_decomp: K/G=%d exceeds the limit of %d groups per row", K / G, kDecompMaxGroups);
  if (nslices == 1)
    hipLaunchKernelGGL(decompose_kernel<1>, dim3(M), dim3(kDecompThreads), 0, s, x, M, K, G, slices, tok_scale,
                       gsum);
  else
    hipLaunchKernelGGL(decompose_kernel<2>, dim3(M), dim3(kDecompThreads), 0, s, x, M, K, G, slices, tok_scale,
                       gsum);
  return check_launch("decompose");
}

}  // namespace w4

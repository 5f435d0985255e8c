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

// One workgroup per token row, passes over the (cache-resident) row: the
// absmax, then slice 1 (with the residual's absmax), then slice 2, whose
// residual is recomputed from x and slice 1 exactly as before.
template <int NS>
__global__ __launch_bounds__(kDecompThreads) void decompose_kernel(
    const uint16_t* __restrict__ x, int M, int K, int G, int8_t* __restrict__ slices,
    float* __restrict__ tok_scale, int32_t* __restrict__ gsum) {
  __shared__ double red[kDecompThreads / kWave];
  __shared__ int gs[NS][kDecompMaxGroups];
  const int m = blockIdx.x;
  const int ng = K / G;
  const uint16_t* xr = x + (size_t)m * K;
  for (int t = threadIdx.x; t < NS * ng; t += kDecompThreads) gs[t / ng][t % ng] = 0;

  double amax = 0.0;
  for (int k = threadIdx.x; k < K; k += kDecompThreads) amax = fmax(amax, fabs((double)half_bits_to_float(xr[k])));
  amax = block_max(amax, red);  // also orders the gs clearing before the atomics below
  const double s1 = (double)(float)(amax / 127.0);

  int8_t* out1 = slices + (size_t)m * K;
  double amax2 = 0.0;
  for (int k = threadIdx.x; k < K; k += kDecompThreads) {
    const double xv = (double)half_bits_to_float(xr[k]);
    const double a = quant127(xv, s1);
    out1[k] = (int8_t)(int)a;
    atomicAdd(&gs[0][k / G], (int)a);
    amax2 = fmax(amax2, fabs(xv - s1 * a));
  }
  if (threadIdx.x == 0) tok_scale[m] = (float)s1;
  if constexpr (NS == 2) {
    amax2 = block_max(amax2, red);
    const double s2 = (double)(float)(amax2 / 127.0);
    int8_t* out2 = slices + ((size_t)M + m) * K;
    for (int k = threadIdx.x; k < K; k += kDecompThreads) {
      const double xv = (double)half_bits_to_float(xr[k]);
      const double r1 = xv - s1 * quant127(xv, s1);
      const double a = quant127(r1, s2);
      out2[k] = (int8_t)(int)a;
      atomicAdd(&gs[1][k / G], (int)a);
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

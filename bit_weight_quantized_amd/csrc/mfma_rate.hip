// Matrix-core issue rate: the measured ceiling the prefill products are
// compared with, beside the nominal dense peak.  Every wave issues a fixed
// number of independent 16 x 16 products (no loads, no LDS, no barriers),
// optionally with V independent fp32 FMAs per product, and records the
// shader-clock and real-time ticks it spent, so one launch gives the rate the
// matrix cores sustain at the clock the part runs under that load, and a
// sweep over V shows how many VALU instructions run beside a product for free.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {
namespace {

constexpr int kRateThreads = 512;  // 8 waves, two per SIMD, as the prefill products
constexpr int kRateAcc = 8;        // independent accumulators per wave
// dynamic LDS reserved (and unused) so that one workgroup runs per CU, as
// with the prefill products' three copy stages
constexpr int kRateLds = 96 * 1024;

template <int KIND, int V>
__global__ __launch_bounds__(kRateThreads) void mfma_rate_kernel(int iters, float* __restrict__ sink,
                                                                 unsigned long long* __restrict__ ticks) {
  const int lane = threadIdx.x % kWave;
  // operands that the compiler cannot fold: small values derived from the lane
  const uint32_t base = 0x3C003C00u ^ (uint32_t)(lane & 7);
  const u32x4 a{base, base ^ 1u, base ^ 2u, base ^ 3u};
  const u32x4 b{base ^ 4u, base ^ 5u, base ^ 6u, base ^ 7u};
  const u32x4 ai{0x01010101u * (uint32_t)(lane & 3), 0x01020304u, 0x02010201u, 0x01000100u};
  f32x4 accf[kRateAcc];
  i32x4 acci[kRateAcc];
#pragma unroll
  for (int j = 0; j < kRateAcc; ++j) {
    accf[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    acci[j] = i32x4{0, 0, 0, 0};
  }
  float f[kRateAcc][V > 0 ? V : 1];
#pragma unroll
  for (int j = 0; j < kRateAcc; ++j)
#pragma unroll
    for (int v = 0; v < (V > 0 ? V : 1); ++v) f[j][v] = (float)(lane + j + v);
  const float fs = 0.999f + 1e-6f * (float)lane, ft = 1e-3f;

  const unsigned long long c0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kRateAcc; ++j) {
      if constexpr (KIND == 0)
        accf[j] = mfma_f16(a, b, accf[j]);
      else
        acci[j] = mfma_i8(ai, ai, acci[j]);
#pragma unroll
      for (int v = 0; v < V; ++v) f[j][v] = fmaf(f[j][v], fs, ft);
    }
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();

  float s = 0.f;
#pragma unroll
  for (int j = 0; j < kRateAcc; ++j) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s += KIND == 0 ? accf[j][i] : (float)acci[j][i];
    if constexpr (V > 0) {
#pragma unroll
      for (int v = 0; v < V; ++v) s += f[j][v];
    }
  }
  const size_t t = (size_t)blockIdx.x * kRateThreads + threadIdx.x;
  sink[t] = s;
  if (ticks && lane == 0) {
    const size_t w = t / kWave;
    ticks[2 * w] = c1 - c0;
    ticks[2 * w + 1] = r1 - r0;
  }
}

template <int KIND, int V>
int launch_rate(int workgroups, int iters, float* sink, unsigned long long* ticks, hipStream_t s) {
  const int st = allow_dynamic_lds(reinterpret_cast<const void*>(&mfma_rate_kernel<KIND, V>), kRateLds, "w4_mfma_rate");
  if (st) return st;
  hipLaunchKernelGGL((mfma_rate_kernel<KIND, V>), dim3((unsigned)workgroups), dim3(kRateThreads), kRateLds, s, iters,
                     sink, ticks);
  return check_launch("mfma_rate");
}

template <int KIND>
int launch_rate_kind(int valu, int workgroups, int iters, float* sink, unsigned long long* ticks, hipStream_t s) {
  switch (valu) {
    case 0: return launch_rate<KIND, 0>(workgroups, iters, sink, ticks, s);
    case 1: return launch_rate<KIND, 1>(workgroups, iters, sink, ticks, s);
    case 2: return launch_rate<KIND, 2>(workgroups, iters, sink, ticks, s);
    case 3: return launch_rate<KIND, 3>(workgroups, iters, sink, ticks, s);
    case 4: return launch_rate<KIND, 4>(workgroups, iters, sink, ticks, s);
    case 6: return launch_rate<KIND, 6>(workgroups, iters, sink, ticks, s);
    case 8: return launch_rate<KIND, 8>(workgroups, iters, sink, ticks, s);
    default: return fail(-1 /* W4_EINVAL */, "w4_mfma_rate: valu must be 0, 1, 2, 3, 4, 6 or 8 (got %d)", valu);
  }
}

}  // namespace

int launch_mfma_rate(int kind, int valu, int workgroups, int iters, float* sink, unsigned long long* ticks,
                     hipStream_t s) {
  return kind == 0 ? launch_rate_kind<0>(valu, workgroups, iters, sink, ticks, s)
                   : launch_rate_kind<1>(valu, workgroups, iters, sink, ticks, s);
}

}  // namespace w4

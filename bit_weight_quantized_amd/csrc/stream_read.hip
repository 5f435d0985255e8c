// Plain read of a device buffer: the HBM read rate the weight-streaming
// kernels are measured against (their weights are read once per call, with
// 16-byte non-temporal loads, the way this kernel reads its buffer).
#include "w4_device.h"
#include "w4_internal.h"

#include <algorithm>

namespace w4 {
namespace {

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 4;  // 16-byte loads in flight per thread

// Thread i folds pieces i, i + T, i + 2T, ... (T = all threads) into an XOR;
// workgroup b's XOR goes to acc[64 (b mod 8)] with one atomic.  Atomics on
// one word serialize (about 9 ns each on MI355X: 1088 of them add 10 us to a
// 7.5 us read); eight words 256 bytes apart cost about 0.4 us.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32x4* __restrict__ p, long n16,
                                                                   uint32_t* __restrict__ acc) {
  __shared__ uint32_t red[kReadThreads / kWave];
  const long nthr = (long)gridDim.x * kReadThreads;
  uint32_t v = 0;
  for (long base = (long)blockIdx.x * kReadThreads + threadIdx.x; base < n16; base += nthr * kReadUnroll) {
    u32x4 w[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const long i = base + (long)u * nthr;
      w[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v ^= w[u].x ^ w[u].y ^ w[u].z ^ w[u].w;
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v ^= (uint32_t)__shfl_xor((int)v, off, kWave);
  if (threadIdx.x % kWave == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < kReadThreads / kWave; ++w) r ^= red[w];
    __hip_atomic_fetch_xor(acc + 64 * (blockIdx.x % 8), r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

int launch_stream_read(const void* buf, size_t bytes, uint32_t* acc, hipStream_t s) {
  const long n16 = (long)(bytes / 16);
  if (n16 == 0) return 0;
  const long per = (long)kReadThreads * kReadUnroll;
  const long blocks = std::min<long>((n16 + per - 1) / per, 1L << 20);
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, s,
                     static_cast<const u32x4*>(buf), n16, acc);
  return check_launch("stream_read");
}

}  // namespace w4

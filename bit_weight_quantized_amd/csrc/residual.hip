// Residual compensation of salient channels ("DecDEC: A Systems Approach to
// Advancing Low-Bit LLM Quantization", Abstract): the residual R = W - W'
// stays in host memory; at each decode step the channels where the
// activations have outliers are picked, and only their residual rows cross
// the host link to correct the quantized product:
//   y[m, n] += sum over picked channels c of x[m, c] * R[c, n].
//
// Salience of channel c: max_m |x[m, c]|; the k highest are picked, ordered by
// score (descending) and channel (ascending).  The residual is fp16,
// channel-major ([K][N]), so one picked channel is one contiguous row.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kIdxBits = 17;  // channel field of a selection key

// ---------------------------------------------------------------------------
// Selection: one workgroup.  Key of channel c = (max_m |x[m, c]| as fp16 bits)
// << 17 | (2^17 - 1 - c); for finite inputs the bit pattern of |x| orders like
// its value, so larger keys are higher scores and, among equal scores, lower
// channels, and keys are distinct (and nonzero, since K < 2^17).  A radix
// select (four 8-bit digits, most significant first) finds the k-th largest
// key T; the k keys >= T are gathered and sorted (bitonic, descending).
__global__ __launch_bounds__(kSelThreads) void salient_select_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                     int k, int32_t* __restrict__ idx) {
  extern __shared__ uint32_t keys[];  // [K]
  __shared__ uint32_t hist[256];
  __shared__ uint32_t top[kSelMaxTop];
  __shared__ uint32_t s_prefix, s_remaining, s_count;
  const int tid = threadIdx.x;

  for (int c = tid; c < K; c += kSelThreads) {
    uint32_t s = 0;
    for (int m = 0; m < M; ++m) s = max(s, (uint32_t)(x[(size_t)m * K + c] & 0x7FFFu));
    keys[c] = (s << kIdxBits) | (uint32_t)((1 << kIdxBits) - 1 - c);
  }
  if (tid == 0) {
    s_prefix = 0;
    s_remaining = (uint32_t)k;
    s_count = 0;
  }
  __syncthreads();

  uint32_t mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int c = tid; c < K; c += kSelThreads) {
      const uint32_t key = keys[c];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // the digit whose bucket holds the remaining-th largest candidate: lane
      // l owns buckets 4l .. 4l + 3; a suffix scan over the lanes gives the
      // count above each lane's buckets, and exactly one lane's range holds
      // the rank (counts over all buckets cover it)
      const uint32_t rem = s_remaining;
      uint32_t h[4], own = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) own += (h[b] = hist[4 * tid + b]);
      uint32_t incl = own;  // sum over lanes >= tid
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t t = __shfl_down(incl, off);
        if (tid + off < kWave) incl += t;
      }
      const uint32_t above = incl - own;
      if (above < rem && rem <= incl) {
        uint32_t r = rem - above;
        int b = 3;
        while (b > 0 && h[b] < r) r -= h[b--];
        s_remaining = r;
        s_prefix = prefix | ((uint32_t)(4 * tid + b) << shift);
      }
    }
    mask |= 255u << shift;
    __syncthreads();
  }

  const uint32_t T = s_prefix;  // the k-th largest key
  for (int c = tid; c < K; c += kSelThreads) {
    const uint32_t key = keys[c];
    if (key >= T) top[atomicAdd(&s_count, 1u)] = key;
  }
  int P = 1;
  while (P < k) P <<= 1;
  for (int i = k + tid; i < P; i += kSelThreads) top[i] = 0;  // padding sorts last
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1)
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < P / 2; i += kSelThreads) {
        const int lo = 2 * i - (i & (stride - 1)), hi = lo + stride;
        const bool desc = (lo & size) == 0;  // the final merge (size = P) is descending
        const uint32_t a = top[lo], b = top[hi];
        if ((a < b) == desc) {
          top[lo] = b;
          top[hi] = a;
        }
      }
      __syncthreads();
    }
  for (int j = tid; j < k; j += kSelThreads)
    idx[j] = (1 << kIdxBits) - 1 - (int)(top[j] & ((1u << kIdxBits) - 1));
}

// ---------------------------------------------------------------------------
// Correction.  A workgroup owns 64 * CPT output columns for every token; its
// 8 waves take the picked channels round-robin (channel j to wave j mod 8),
// each lane reading CPT residuals of a row (one 16-byte or 4-byte load, a
// wave one contiguous 1 KB or 256 B piece of the row) straight from host
// memory, four channels' loads in flight at a time.  The waves' fp32 partial
// sums meet in LDS and are added in wave order, then to y once.
constexpr int kCorrWaves = 8;
constexpr int kCorrBatch = 4;

template <int CPT, int MMAX>
__global__ __launch_bounds__(kCorrWaves * kWave) void residual_correct_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint16_t* __restrict__ resid,
    const int32_t* __restrict__ idx, int k, uint16_t* __restrict__ y) {
  extern __shared__ float part[];  // [kCorrWaves][MMAX][64 * CPT]
  constexpr int kCols = 64 * CPT;
  const int lane = threadIdx.x % kWave;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int n = blockIdx.x * kCols + lane * CPT;  // this lane's first column
  const bool in_n = n < N;                        // N % CPT == 0

  float acc[MMAX][CPT];
#pragma unroll
  for (int m = 0; m < MMAX; ++m)
#pragma unroll
    for (int i = 0; i < CPT; ++i) acc[m][i] = 0.f;

  for (int j0 = w; j0 < k; j0 += kCorrWaves * kCorrBatch) {
    int c[kCorrBatch];
    float r[kCorrBatch][CPT];
#pragma unroll
    for (int b = 0; b < kCorrBatch; ++b) {
      const int j = j0 + b * kCorrWaves;
      const int cc = j < k ? idx[j] : -1;
      c[b] = (unsigned)cc < (unsigned)K ? cc : -1;  // entries outside [0, K) are skipped
      const uint16_t* row = resid + (size_t)(c[b] < 0 ? 0 : c[b]) * N + (in_n ? n : 0);
      if constexpr (CPT == 8) {
        const u32x4 v = c[b] >= 0 ? *reinterpret_cast<const u32x4*>(row) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          r[b][2 * i] = half_bits_to_float((uint16_t)(v[i] & 0xFFFFu));
          r[b][2 * i + 1] = half_bits_to_float((uint16_t)(v[i] >> 16));
        }
      } else {
        const uint32_t v = c[b] >= 0 ? *reinterpret_cast<const uint32_t*>(row) : 0u;
        r[b][0] = half_bits_to_float((uint16_t)(v & 0xFFFFu));
        r[b][1] = half_bits_to_float((uint16_t)(v >> 16));
      }
    }
#pragma unroll
    for (int b = 0; b < kCorrBatch; ++b) {
      if (c[b] < 0) continue;
#pragma unroll
      for (int m = 0; m < MMAX; ++m) {
        if (m < M) {
          const float xv = half_bits_to_float(x[(size_t)m * K + c[b]]);
#pragma unroll
          for (int i = 0; i < CPT; ++i) acc[m][i] = fmaf(xv, r[b][i], acc[m][i]);
        }
      }
    }
  }

#pragma unroll
  for (int m = 0; m < MMAX; ++m)
#pragma unroll
    for (int i = 0; i < CPT; ++i) part[(w * MMAX + m) * kCols + lane * CPT + i] = acc[m][i];
  __syncthreads();
  for (int o = threadIdx.x; o < M * kCols; o += kCorrWaves * kWave) {
    const int m = o / kCols, col = o % kCols, nn = blockIdx.x * kCols + col;
    if (nn >= N) continue;
    float s = 0.f;
    for (int ww = 0; ww < kCorrWaves; ++ww) s += part[(ww * MMAX + m) * kCols + col];
    const size_t at = (size_t)m * N + nn;
    y[at] = float_to_half_bits(half_bits_to_float(y[at]) + s);
  }
}

template <int CPT, int MMAX>
int launch_correct_t(const uint16_t* x, int M, int K, int N, const uint16_t* resid, const int32_t* idx, int k,
                     uint16_t* y, hipStream_t s) {
  const int lds = kCorrWaves * MMAX * 64 * CPT * (int)sizeof(float);
  const void* fn = reinterpret_cast<const void*>(&residual_correct_kernel<CPT, MMAX>);
  const int st = allow_dynamic_lds(fn, lds, "w4_residual_correct");
  if (st != 0) return st;
  const int blocks = (N + 64 * CPT - 1) / (64 * CPT);
  hipLaunchKernelGGL((residual_correct_kernel<CPT, MMAX>), dim3(blocks), dim3(kCorrWaves * kWave), lds, s, x, M, K,
                     N, resid, idx, k, y);
  return check_launch("residual_correct");
}

}  // namespace

int launch_salient_select(const uint16_t* x, int M, int K, int k, int32_t* idx, hipStream_t s) {
  const int lds = K * (int)sizeof(uint32_t);
  const void* fn = reinterpret_cast<const void*>(&salient_select_kernel);
  const int st = allow_dynamic_lds(fn, lds, "w4_salient_select");
  if (st != 0) return st;
  hipLaunchKernelGGL(salient_select_kernel, dim3(1), dim3(kSelThreads), lds, s, x, M, K, k, idx);
  return check_launch("salient_select");
}

int launch_residual_correct(const uint16_t* x, int M, int K, int N, const uint16_t* resid, const int32_t* idx,
                            int k, uint16_t* y, hipStream_t s) {
  if (M <= 8) return launch_correct_t<8, 8>(x, M, K, N, resid, idx, k, y, s);
  return launch_correct_t<2, 32>(x, M, K, N, resid, idx, k, y, s);
}

}  // namespace w4

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
// select (8-bit digits, most significant first) narrows down the prefix of
// the k-th largest key; it stops as soon as the bucket holding that key holds
// exactly the keys still needed, so every key whose prefix is at least the
// final prefix is picked (usually after two digits).  The k picked keys are
// gathered (one atomic per wave) and each is written to the place its rank
// among them gives (the number of larger keys), which is the sorted order.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// LDS of one selection: keys[K] (caller-sized), hist[256], top[kSelMaxTop]
// and four scalars; idx (LDS or device memory) receives the k channels.
struct SelLds {
  uint32_t hist[256];
  __align__(16) uint32_t top[kSelMaxTop];
  uint32_t prefix, remaining, count, done;
};

template <int NT>
__device__ void select_salient(const uint16_t* __restrict__ x, int M, int K, int k, uint32_t* keys, SelLds& sl,
                               int32_t* idx) {
  uint32_t* hist = sl.hist;
  uint32_t* top = sl.top;
  uint32_t& s_prefix = sl.prefix;
  uint32_t& s_remaining = sl.remaining;
  uint32_t& s_count = sl.count;
  uint32_t& s_done = sl.done;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;

  // keys: thread t scores channels 8 t .. 8 t + 7 of each chunk of 8 NT,
  // with the loads of four rows in flight at a time (16-byte loads when x
  // and K allow them; otherwise eight 2-byte loads, the index clamped to the
  // row so that none is conditional)
  auto store_keys = [&](int c0, const uint32_t (&mx)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (c0 + e < K) keys[c0 + e] = (mx[e] << kIdxBits) | (uint32_t)((1 << kIdxBits) - 1 - (c0 + e));
  };
  auto fold = [](uint32_t (&mx)[8], const u32x4& v) {
#pragma unroll
    for (int e = 0; e < 8; ++e) mx[e] = max(mx[e], (v[e / 2] >> (16 * (e % 2))) & 0x7FFFu);
  };
  if ((reinterpret_cast<uintptr_t>(x) & 15u) == 0 && K % 8 == 0) {
    for (int c0 = 8 * tid; c0 < K; c0 += 8 * NT) {
      uint32_t mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int m0 = 0; m0 < M; m0 += 4) {
        u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          v[u] = m0 + u < M ? *reinterpret_cast<const u32x4*>(x + (size_t)(m0 + u) * K + c0) : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) fold(mx, v[u]);
      }
      store_keys(c0, mx);
    }
  } else {
    for (int c0 = 8 * tid; c0 < K; c0 += 8 * NT) {
      uint32_t mx[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      for (int m0 = 0; m0 < M; m0 += 4) {
        uint16_t h[4][8];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const uint16_t* row = x + (size_t)min(m0 + u, M - 1) * K;
#pragma unroll
          for (int e = 0; e < 8; ++e) h[u][e] = row[min(c0 + e, K - 1)];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          u32x4 v{0, 0, 0, 0};
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (m0 + u < M && c0 + e < K) v[e / 2] |= (uint32_t)h[u][e] << (16 * (e % 2));
          fold(mx, v);
        }
      }
      store_keys(c0, mx);
    }
  }
  if (tid == 0) {
    s_prefix = 0;
    s_remaining = (uint32_t)k;
    s_count = 0;
    s_done = 0;
  }
  __syncthreads();

  uint32_t mask = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    const uint32_t prefix = s_prefix;
    for (int c = tid; c < K; c += NT) {
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
        if (h[b] == r) s_done = 1;  // the whole bucket is needed: its keys and every larger one
      }
    }
    mask |= 255u << shift;
    __syncthreads();
    if (s_done) break;
  }

  // gather the k keys whose masked prefix is at least the final prefix
  const uint32_t T = s_prefix;
  for (int c0 = 0; c0 < K; c0 += NT) {  // wave-uniform trip count
    const int c = c0 + tid;
    const uint32_t key = c < K ? keys[c] : 0u;
    const bool sel = c < K && (key & mask) >= T;
    const uint64_t b = __ballot(sel);
    if (b) {
      uint32_t base = 0;
      if (lane == 0) base = atomicAdd(&s_count, (uint32_t)__popcll(b));
      base = (uint32_t)__shfl((int)base, 0);
      if (sel) top[base + lanes_below(b)] = key;
    }
  }
  // zeros after the k keys up to a multiple of 8 (every key is at least 1:
  // its low bits are 2^17 - 1 - c with c < 2^17), so the rank loop below
  // reads whole 16-byte pieces
  const int k8 = (k + 7) & ~7;  // <= kSelMaxTop
  if (tid < k8 - k) top[k + tid] = 0u;
  __syncthreads();
  // rank of each gathered key = number of larger ones (keys are distinct);
  // the reads are the same for every lane (broadcast), eight keys per step
  for (int i = tid; i < k; i += NT) {
    const uint32_t key = top[i];
    int r = 0;
#pragma unroll 4
    for (int j = 0; j < k8; j += 8) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(top + j);
      const u32x4 b = *reinterpret_cast<const u32x4*>(top + j + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) r += (a[e] > key ? 1 : 0) + (b[e] > key ? 1 : 0);
    }
    idx[r] = (1 << kIdxBits) - 1 - (int)(key & ((1u << kIdxBits) - 1));
  }
}

__global__ __launch_bounds__(kSelThreads) void salient_select_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                                     int k, int32_t* __restrict__ idx) {
  extern __shared__ uint32_t keys[];  // [K]
  __shared__ SelLds sl;
  select_salient<kSelThreads>(x, M, K, k, keys, sl, idx);
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

// F32: the correction is stored to c (fp32 [M][N]) instead of added to y.
template <int CPT, int MMAX, bool F32>
__device__ void correct_columns(const uint16_t* __restrict__ x, int M, int K, int N, const uint16_t* __restrict__ resid,
                                const int32_t* idx, int k, uint16_t* __restrict__ y, float* __restrict__ c,
                                float* part) {
  // part: LDS [kCorrWaves][MMAX][64 * CPT]
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
    if constexpr (F32) c[at] = s;
    else y[at] = float_to_half_bits(half_bits_to_float(y[at]) + s);
  }
}

template <int CPT, int MMAX, bool F32>
__global__ __launch_bounds__(kCorrWaves * kWave) void residual_correct_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint16_t* __restrict__ resid,
    const int32_t* __restrict__ idx, int k, uint16_t* __restrict__ y, float* __restrict__ c) {
  extern __shared__ float part[];  // [kCorrWaves][MMAX][64 * CPT]
  correct_columns<CPT, MMAX, F32>(x, M, K, N, resid, idx, k, y, c, part);
}

// y[i] = fp16(y[i] + c[i]) for i < n (n % 8 == 0), eight elements per thread:
// the same rounding as the correction that adds to y itself.
__global__ __launch_bounds__(256) void residual_apply_kernel(const float* __restrict__ c, size_t n,
                                                             uint16_t* __restrict__ y) {
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const u32x4 yv = *reinterpret_cast<const u32x4*>(y + i);
  const float4 c0 = *reinterpret_cast<const float4*>(c + i), c1 = *reinterpret_cast<const float4*>(c + i + 4);
  const float cv[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
  u32x4 out;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint16_t lo = float_to_half_bits(half_bits_to_float((uint16_t)(yv[j] & 0xFFFFu)) + cv[2 * j]);
    const uint16_t hi = float_to_half_bits(half_bits_to_float((uint16_t)(yv[j] >> 16)) + cv[2 * j + 1]);
    out[j] = (uint32_t)lo | ((uint32_t)hi << 16);
  }
  *reinterpret_cast<u32x4*>(y + i) = out;
}

// Selection and correction in one launch: every workgroup picks the channels
// itself (the same ones: the selection is deterministic) into LDS, workgroup 0
// also writes them to idx, and each then corrects its columns.  The dynamic
// LDS holds the selection keys first and the correction's partial sums after.
template <int CPT, int MMAX, bool F32>
__global__ __launch_bounds__(kCorrWaves * kWave) void salient_correct_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint16_t* __restrict__ resid, int k,
    int32_t* __restrict__ idx, uint16_t* __restrict__ y, float* __restrict__ c) {
  extern __shared__ uint32_t dyn[];  // keys[K], then part[kCorrWaves][MMAX][64 * CPT]
  __shared__ SelLds sl;
  __shared__ int32_t picked[kSelMaxTop];
  select_salient<kCorrWaves * kWave>(x, M, K, k, dyn, sl, picked);
  __syncthreads();
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < k; i += kCorrWaves * kWave) idx[i] = picked[i];
  correct_columns<CPT, MMAX, F32>(x, M, K, N, resid, picked, k, y, c, reinterpret_cast<float*>(dyn));
}

template <int CPT, int MMAX, bool F32>
int launch_correct_t(const uint16_t* x, int M, int K, int N, const uint16_t* resid, const int32_t* idx, int k,
                     uint16_t* y, float* c, hipStream_t s) {
  const int lds = kCorrWaves * MMAX * 64 * CPT * (int)sizeof(float);
  const void* fn = reinterpret_cast<const void*>(&residual_correct_kernel<CPT, MMAX, F32>);
  const int st = allow_dynamic_lds(fn, lds, F32 ? "w4_residual_correct_f32" : "w4_residual_correct");
  if (st != 0) return st;
  const int blocks = (N + 64 * CPT - 1) / (64 * CPT);
  hipLaunchKernelGGL((residual_correct_kernel<CPT, MMAX, F32>), dim3(blocks), dim3(kCorrWaves * kWave), lds, s, x, M,
                     K, N, resid, idx, k, y, c);
  return check_launch(F32 ? "residual_correct_f32" : "residual_correct");
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
  if (M <= 8) return launch_correct_t<8, 8, false>(x, M, K, N, resid, idx, k, y, nullptr, s);
  return launch_correct_t<2, 32, false>(x, M, K, N, resid, idx, k, y, nullptr, s);
}

int launch_residual_correct_f32(const uint16_t* x, int M, int K, int N, const uint16_t* resid, const int32_t* idx,
                                int k, float* c, hipStream_t s) {
  if (M <= 8) return launch_correct_t<8, 8, true>(x, M, K, N, resid, idx, k, nullptr, c, s);
  return launch_correct_t<2, 32, true>(x, M, K, N, resid, idx, k, nullptr, c, s);
}

int launch_residual_apply(const float* c, int M, int N, uint16_t* y, hipStream_t s) {
  const size_t n = (size_t)M * N;
  const unsigned blocks = (unsigned)((n / 8 + 255) / 256);
  hipLaunchKernelGGL(residual_apply_kernel, dim3(blocks), dim3(256), 0, s, c, n, y);
  return check_launch("residual_apply");
}

template <int CPT, int MMAX, bool F32>
int launch_salient_correct_t(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k, int32_t* idx,
                             uint16_t* y, float* c, hipStream_t s) {
  const int lds = std::max(K * (int)sizeof(uint32_t), kCorrWaves * MMAX * 64 * CPT * (int)sizeof(float));
  const void* fn = reinterpret_cast<const void*>(&salient_correct_kernel<CPT, MMAX, F32>);
  const int st = allow_dynamic_lds(fn, lds, F32 ? "w4_salient_correct_f32" : "w4_salient_correct");
  if (st != 0) return st;
  const int blocks = (N + 64 * CPT - 1) / (64 * CPT);
  hipLaunchKernelGGL((salient_correct_kernel<CPT, MMAX, F32>), dim3(blocks), dim3(kCorrWaves * kWave), lds, s, x, M,
                     K, N, resid, k, idx, y, c);
  return check_launch(F32 ? "salient_correct_f32" : "salient_correct");
}

int launch_salient_correct(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k, int32_t* idx,
                           uint16_t* y, hipStream_t s) {
  if (M <= 8) return launch_salient_correct_t<8, 8, false>(x, M, K, N, resid, k, idx, y, nullptr, s);
  return launch_salient_correct_t<2, 32, false>(x, M, K, N, resid, k, idx, y, nullptr, s);
}

int launch_salient_correct_f32(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k, int32_t* idx,
                               float* c, hipStream_t s) {
  if (M <= 8) return launch_salient_correct_t<8, 8, true>(x, M, K, N, resid, k, idx, nullptr, c, s);
  return launch_salient_correct_t<2, 32, true>(x, M, K, N, resid, k, idx, nullptr, c, s);
}

}  // namespace w4

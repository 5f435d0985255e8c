// Offline weight preparation: INT4 asymmetric and NF4 quantization, nibble
// packing.  Bit-exact by construction: every decision is taken in fp64 with
// IEEE operations (no contraction), and the fp64 -> fp32 -> fp16 roundings are
// explicit round-to-nearest-even conversions.
//
// INT4 asymmetric: one scale and one zero point per group ("MixPE:
// Quantization and Hardware Co-design for Efficient LLM Inference", Abstract).
// NF4: 16-level NormalFloat codebook with a per-block absmax ("Fast NF4
// Dequantization Kernels for Large Language Model Inference", Abstract).
#include "w4_device.h"
#include "w4_internal.h"

#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int kQuantWavesPerBlock = 4;

// One wave per (row n, group g).  Lane i holds elements i, i+64, ... of the
// group.  The group's min and max (exact in fp32) are reduced across the wave,
// then each lane applies the fp64 steps to its own elements.
template <int G>
__global__ __launch_bounds__(kWave * kQuantWavesPerBlock) void quantize_int4_kernel(
    const float* __restrict__ wt, int K, long n_groups, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scale, uint16_t* __restrict__ zero) {
  constexpr int E = G / kWave;
  const int lane = threadIdx.x % kWave;
  const long grp = (long)blockIdx.x * kQuantWavesPerBlock + threadIdx.x / kWave;
  if (grp >= n_groups) return;
  const int ng = K / G;
  const long n = grp / ng;
  const int g = (int)(grp % ng);
  const float* src = wt + n * (long)K + (long)g * G;
  float w[E];
  float mn = 0.0f, mx = 0.0f;  // lo = min(0, min w), hi = max(0, max w)
#pragma unroll
  for (int e = 0; e < E; ++e) {
    w[e] = src[lane + kWave * e];
    mn = fminf(mn, w[e]);
    mx = fmaxf(mx, w[e]);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  const double lo = (double)mn, hi = (double)mx;
  const float s32 = (float)((hi - lo) / 15.0);
  const uint16_t s16 = float_to_half_bits(s32);
  const double s = (double)half_bits_to_float(s16);
  double z = 0.0;
  if (s != 0.0) z = fmin(fmax(rint(-lo / s), 0.0), 15.0) + 0.0;
  uint8_t* dst = codes + n * (long)K + (long)g * G;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    double q = 0.0;
    if (s != 0.0) q = fmin(fmax(rint((double)w[e] / s) + z, 0.0), 15.0);
    dst[lane + kWave * e] = (uint8_t)(int)q;
  }
  if (lane == 0) {
    scale[grp] = s16;
    zero[grp] = float_to_half_bits((float)z);
  }
}

// One wave per (row n, block b): a = fp16(max|w|); code = lowest index of the
// nearest level c_i * a, compared in fp64 (c_i * a is exact).
template <int B>
__global__ __launch_bounds__(kWave * kQuantWavesPerBlock) void quantize_nf4_kernel(
    const float* __restrict__ wt, int K, long n_blocks, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ absmax) {
  constexpr int E = B / kWave;
  const int lane = threadIdx.x % kWave;
  const long blk = (long)blockIdx.x * kQuantWavesPerBlock + threadIdx.x / kWave;
  if (blk >= n_blocks) return;
  const int nb = K / B;
  const long n = blk / nb;
  const int b = (int)(blk % nb);
  const float* src = wt + n * (long)K + (long)b * B;
  float w[E];
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    w[e] = src[lane + kWave * e];
    amax = fmaxf(amax, fabsf(w[e]));
  }
  amax = wave_max(amax);
  const uint16_t a16 = float_to_half_bits(amax);
  const double a = (double)half_bits_to_float(a16);
  uint8_t* dst = codes + n * (long)K + (long)b * B;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    int best = 7;
    if (a != 0.0) {
      const double wv = (double)w[e];
      best = 0;
      double bestd = fabs(wv - (double)nf4_level(0) * a);
      for (int i = 1; i < 16; ++i) {
        const double d = fabs(wv - (double)nf4_level(i) * a);
        if (d < bestd) {  // strict: ties keep the lower index
          bestd = d;
          best = i;
        }
      }
    }
    dst[lane + kWave * e] = (uint8_t)best;
  }
  if (lane == 0) absmax[blk] = a16;
}

// Stored form of the packed weights: tiles of 16 rows x 128 K positions,
// tile (nb, kb) = rows 16 nb .. 16 nb + 15 x K positions 128 kb .. 128 kb + 127,
// 1024 contiguous bytes at (nb * K / 128 + kb) * 1024.  "Lane" l = 16 j + r of
// a tile owns bytes 16 l .. 16 l + 15: little-endian word t holds the 8 codes
// of row r at K positions 32 t + 8 j + 0..7, the even positions in nibbles
// 0-3 and the odd ones in nibbles 4-7 (nibble p: position 0,2,4,6,1,3,5,7).
// One 16-byte load per lane of a wave therefore delivers a whole tile in the
// operand order of the 16x16 matrix-core products, and the masks
// (w >> 4 i) & 0x000F000F produce the fp16 pairs (c_2i, c_2i+1) in K order.
//
// One thread per 16-byte lane slot: four 8-byte code loads, 16 bytes out.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ codes, int K,
                                                   long n_slots, uint8_t* __restrict__ packed) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n_slots) return;
  const int kt = K / 128;
  const long tile = idx / 64;
  const int l = (int)(idx % 64);
  const long nb = tile / kt;
  const int kb = (int)(tile % kt);
  const int r = l % 16, j = l / 16;
  const uint8_t* row = codes + (nb * 16 + r) * (long)K + kb * 128 + 8 * j;
  uint32_t out[4];
  // four codes (one per byte, each < 16) -> four nibbles, first code lowest
  auto nib4 = [](uint32_t v) {
    const uint32_t p = (v | (v >> 4)) & 0x00FF00FFu;
    return (p & 0xFFu) | ((p >> 8) & 0xFF00u);
  };
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const u32x2 c = *reinterpret_cast<const u32x2*>(row + 32 * t);  // codes k .. k + 7, one per byte
    const uint32_t even = perm_b32(c.y, c.x, 0x06040200u) & 0x0F0F0F0Fu;  // c0 c2 c4 c6
    const uint32_t odd = perm_b32(c.y, c.x, 0x07050301u) & 0x0F0F0F0Fu;   // c1 c3 c5 c7
    out[t] = nib4(even) | (nib4(odd) << 16);
  }
  reinterpret_cast<u32x4*>(packed)[idx] = u32x4{out[0], out[1], out[2], out[3]};
}

}  // namespace

int launch_quantize_int4(const float* wt, int K, int N, int G, uint8_t* codes,
                         uint16_t* scale, uint16_t* zero, hipStream_t s) {
  const long n_groups = (long)N * (K / G);
  if (n_groups == 0) return 0;
  const dim3 grid((unsigned)((n_groups + kQuantWavesPerBlock - 1) / kQuantWavesPerBlock));
  const dim3 block(kWave * kQuantWavesPerBlock);
  if (G == 64)
    hipLaunchKernelGGL(quantize_int4_kernel<64>, grid, block, 0, s, wt, K, n_groups, codes, scale, zero);
  else
    hipLaunchKernelGGL(quantize_int4_kernel<128>, grid, block, 0, s, wt, K, n_groups, codes, scale, zero);
  return check_launch("quantize_int4");
}

int launch_quantize_nf4(const float* wt, int K, int N, int G, uint8_t* codes,
                        uint16_t* absmax, hipStream_t s) {
  const long n_blocks = (long)N * (K / G);
  if (n_blocks == 0) return 0;
  const dim3 grid((unsigned)((n_blocks + kQuantWavesPerBlock - 1) / kQuantWavesPerBlock));
  const dim3 block(kWave * kQuantWavesPerBlock);
  if (G == 64)
    hipLaunchKernelGGL(quantize_nf4_kernel<64>, grid, block, 0, s, wt, K, n_blocks, codes, absmax);
  else
    hipLaunchKernelGGL(quantize_nf4_kernel<128>, grid, block, 0, s, wt, K, n_blocks, codes, absmax);
  return check_launch("quantize_nf4");
}

int launch_pack(const uint8_t* codes, int K, int N, uint8_t* packed, hipStream_t s) {
  const long n_slots = (long)N * K / 32;  // 16 bytes = 32 codes each
  if (n_slots == 0) return 0;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)((n_slots + 255) / 256)), dim3(256), 0, s, codes, K, n_slots, packed);
  return check_launch("pack");
}

}  // namespace w4

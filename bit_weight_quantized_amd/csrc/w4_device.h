// Device-side helpers for gfx950 (CDNA4, wave64): vector types, matrix-core
// wrappers, wave reductions, fp16 bit helpers and the NF4 level table.
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

namespace w4 {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// NormalFloat levels rounded to fp32 (QLoRA's construction, which the
// "Fast NF4 Dequantization Kernels" page builds on), as bit patterns.
#define W4_NF4_LEVEL_BITS                                                  \
  0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu,          \
      0xbe3d353du, 0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu,      \
      0x3e7c04dau, 0x3ead0336u, 0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u,      \
      0x3f800000u

__device__ __forceinline__ float nf4_level(int i) {
  constexpr uint32_t bits[16] = {W4_NF4_LEVEL_BITS};
  return __uint_as_float(bits[i]);
}

// 16x16x32 fp16 matrix-core product, fp32 accumulate.
// Lane l supplies A[m = l%16][k = 8*(l/16) + i] and B[k = 8*(l/16) + i][n = l%16]
// for i = 0..7, and holds D[m = 4*(l/16) + r][n = l%16], r = 0..3.
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, a),
                                                __builtin_bit_cast(half8, b), c, 0, 0, 0);
}

// 16x16x64 int8 matrix-core product, int32 accumulate; same lane mapping with
// 16 k values per lane (k = 16*(l/16) + i).
__device__ __forceinline__ i32x4 mfma_i8(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a),
                                               __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// Raw buffer access.  The descriptor covers [base, base + bytes); loads at
// offsets past `bytes` return zeros instead of touching memory.
constexpr int kBufferFlags = 0x00020000;  // descriptor word 3 for gfx9 raw buffers
constexpr int kNonTemporal = 2;           // cache-policy bit: streaming (nt)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal);
}
// The same with the default cache policy (data that other waves read again).
__device__ __forceinline__ u32x4 buffer_load16_cached(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
}

typedef __attribute__((address_space(3))) void lds_void;

// Workgroup barrier for the copy pipelines: this wave's LDS reads have
// completed (lgkmcnt(0)) and no memory access moves across it, but its
// global -> LDS copies stay in flight (no vmcnt wait; every wave waits for its
// own copies of a step explicitly before the barrier that publishes them).
// __syncthreads() would also drain the copies of the steps ahead.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// 16 bytes per lane from a raw buffer (offset = voff + soff) to lds_base +
// 16 * lane (lds_base wave-uniform).  Lanes whose voff lies past the buffer
// write zeros.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              unsigned char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}

// Output tile (row block mb, column block nb) of workgroup b among tiles =
// tiles_m x tiles_n.  Workgroups are dealt to the 8 XCDs round-robin; they are
// renumbered so each XCD gets a contiguous run of tiles, and the run walks
// groups of gm row blocks column block by column block: the workgroups that
// run at once on one XCD share gm row blocks of activations and about
// 32 / gm column blocks of weights in that XCD's L2 (gm = 1: one row block,
// every weight block read once per tile).
// The two halves: xcd_run gives workgroup b's place in the launch's
// XCD-contiguous order, tile_mn the tile at a place of the grouped walk.  A
// launch that covers places [p0, p0 + tiles) of a larger walk (the split-K
// tail of a GEMM) maps workgroup b to tile_mn(p0 + xcd_run(b, tiles)).
__device__ __forceinline__ int xcd_run(int b, int tiles) {
  const int xcd = b % 8, idx = b / 8;
  const int per = tiles / 8, rem = tiles % 8;
  return (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
}
__device__ __forceinline__ void tile_mn(int logical, int tiles_m, int tiles_n, int gm, int& mb, int& nb) {
  const int group = logical / (gm * tiles_n);
  const int first = group * gm;
  const int g = min(tiles_m - first, gm);
  const int in = logical - group * gm * tiles_n;
  mb = first + in % g;
  nb = in / g;
}
__device__ __forceinline__ void tile_of(int b, int tiles, int tiles_m, int tiles_n, int gm, int& mb, int& nb) {
  tile_mn(xcd_run(b, tiles), tiles_m, tiles_n, gm, mb, nb);
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fminf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmax(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  return __half_as_ushort(__float2half_rn(f));
}

// clamp(rint(fl64(n / s)), -127, 127) for an exactly known fp64 numerator n
// (x itself, a residual, or 254 times one) and a scale s that is an fp32
// value, decided in fp32.  inv = fl32(1 / s) (the quotient in fp64, so its
// relative error is at most 2^-24 + 2^-53); with nf = fl32(n) the estimate
// t = fl32(nf * inv) is within 3 * 2^-24 * 127.0001 < 2^-15.4 of n / s, since
// every quotient here has |n / s| <= 127.0001.  Where t is at least 2^-14 from
// every half-integer, rint(t) is the decision.  Nearer (about 1 in 8000), the
// sign of n - h s (h the half-integer next to rint(t) on t's side, the only
// one that can lie between t and the quotient), from one fp64 fma of exact
// operands rounded once, says which side the quotient lies on (on h: to
// even).  That decides rint of the exact quotient; rint(fl64(n / s)) is the
// same integer because no quotient here comes within 2^-25 of a half-integer
// without being one (n - h s is a multiple of the finer of the grids of n and
// s / 2, and that grid is at least 2^-25 s wherever the quotient is near a
// half-integer of magnitude 1/2 or more), while fl64 moves a quotient by at
// most 2^-46.  rint is the fp32 addition of 1.5 * 2^23 (ties to even).
constexpr float kRintMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kNearHalf = 0x1p-14f;

__device__ __forceinline__ float decide127(double n, double s, float inv) {
#pragma clang fp contract(off)
  const float t = (float)n * inv;
  float q = (t + kRintMagic) - kRintMagic;
  if (fabsf(fabsf(t - q) - 0.5f) < kNearHalf) {
    const float sg = t >= q ? 1.f : -1.f;
    const double d = fma(-(double)(q + 0.5f * sg), s, n);
    if (d * (double)sg > 0.0 || (d == 0.0 && ((int)q & 1) != 0)) q += sg;
  }
  return fminf(fmaxf(q, -127.f), 127.f);
}

// The fast form of decide127's estimate: rint(fl32(n * inv)) (v_rndne: the
// same integer as the 1.5 * 2^23 addition), with |t - rint(t)| folded into
// dmax.  Since |t - rint(t)| <= 1/2, t lies within 2^-14 of a half-integer
// exactly when that distance exceeds 1/2 - 2^-14 (both sides exact in fp32):
// callers decide a group of values this way and take decide127 for the whole
// group when near127(dmax).  Branch-free.  For |n / s| <= 127.0001 the
// result is in [-127, 127] without a clamp.
__device__ __forceinline__ float rint127_fast(float n, float inv, float& dmax) {
#pragma clang fp contract(off)
  const float t = n * inv;
  const float q = __builtin_rintf(t);
  dmax = fmaxf(dmax, fabsf(t - q));
  return q;
}
__device__ __forceinline__ bool near127(float dmax) { return dmax > 0.5f - kNearHalf; }


}  // namespace w4

// Decode attention over an INT4 KV cache with Multi-Scale Dequant on both
// products ("Multi-Scale Dequant: Eliminating Dequantization Bottleneck via
// Activation Decomposition for Efficient LLM Inference", Abstract: the KV
// cache stays quantized and the other operand of each product is decomposed,
// which cuts the cache's HBM traffic).
//
// Per batch row b and key/value head h, with its G query heads (grouped-query
// attention) as the 16 rows of the matrix-core products:
//  * K [L][d] is INT4 with one scale and zero per token, stored in the
//    library's weight tiles (N = L tokens, K = d = 128): one 1 KB tile per 16
//    tokens.  The queries arrive as two int8 slices (the decomposition
//    kernel); score[g, t] = sK[t] sum_j s_j[g] sum_d A_j[g, d] (qK - zK[t]),
//    the integer sums on the int8 matrix cores with the zero point folded
//    into the weight bytes, scaled by 1/sqrt(d).
//  * Softmax per chunk of 256 positions (flash decoding): chunk max m_c, sum
//    l_c of p = exp(score - m_c).
//  * Values: w = p sV[t] is split per row over the chunk into two int8 slices
//    (B_j, r_j); V^T [d][L] is stored in weight tiles (N = d, K = L), so
//    E_j[g, n] = sum_t B_j[g, t] qV[n, t] runs on the int8 matrix cores, and
//    the zero points enter once per row: o = sum_j r_j (E_j - sum_t B_j zV).
//  * A second kernel combines the chunks: o = sum_c e^(m_c - m) o_c /
//    sum_c e^(m_c - m) l_c.
#include "w4_device.h"
#include "w4_internal.h"

#include <cstdlib>

namespace w4 {
namespace {

constexpr int kHeadDim = 128;
constexpr int kChunk = 256;
constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kAttnWaves = kAttnThreads / kWave;
// Scores are kept in base-2 units, scaled by log2(e) / sqrt(128), so that
// every exponential of the softmax and of the combination is one exp2 (e^x
// = 2^(x log2 e)); the maxima stored with the partials are in the same units.
constexpr float kScoreScale = 0x1.0527dbd87e24dp-3f;  // 0.12751743082459868

__device__ __forceinline__ i32x4 mfma_i8_16x16x64(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// How a row reduction combines: a float maximum, a sum, or the maximum of
// non-negative floats taken on their bits (an integer maximum orders them
// like the values and, unlike the float one, needs no NaN canonicalisation,
// so the DPP move folds into it as it does into the sum).
enum RowOp { kRowMax, kRowSum, kRowMaxNonNeg };

// all-reduce over the 16 lanes of a DPP row (the lanes holding one row group
// of a matrix-core output): swap within pairs and quads, then the row's
// half-mirror (lane i with 7 - i) and mirror (lane i with 15 - i).  Every
// lane's source is in its row, so bound_ctrl changes nothing; it lets the
// compiler fold the move into the add or integer max (one instruction a
// step).
template <RowOp OP>
__device__ __forceinline__ float row16(float v) {
  auto step = [](int x, int ctrl) {
    switch (ctrl) {  // the control must be a constant
      case 0:
        return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, true);  // [1,0,3,2]
      case 1:
        return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, true);  // [2,3,0,1]
      case 2:
        return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, true);  // half mirror
      default:
        return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, true);  // mirror
    }
  };
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int o = step(__builtin_bit_cast(int, v), c);
    if constexpr (OP == kRowMaxNonNeg)
      v = __builtin_bit_cast(float, max(__builtin_bit_cast(uint32_t, v), (uint32_t)o));
    else if constexpr (OP == kRowSum)
      v = v + __builtin_bit_cast(float, o);
    else
      v = fmaxf(v, __builtin_bit_cast(float, o));
  }
  return v;
}

// reduces NV arrays of 4 row values (rows 4 kb + i of the lane) over the 16
// lanes of a row group and then over the waves through the LDS buffer red;
// array a is a max when bit a of MAXMASK is set, else a sum (integer sums go
// through float, exact below 2^24).  One barrier: the caller alternates
// between two buffers, so the barrier of the previous reduction, which every
// wave reaches only after reading that reduction's buffer, already ordered
// the reads of the buffer written here.
template <int MAXMASK, int NV>
__device__ __forceinline__ void reduce_rows(float (&v)[NV][4], float* red, int w, int lane) {
#pragma unroll
  for (int a = 0; a < NV; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) v[a][i] = ((MAXMASK >> a) & 1) ? row16<kRowMax>(v[a][i]) : row16<kRowSum>(v[a][i]);
  if (lane % 16 == 0)
#pragma unroll
    for (int a = 0; a < NV; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(a * kAttnWaves + w) * 16 + 4 * (lane / 16) + i] = v[a][i];
  __syncthreads();
#pragma unroll
  for (int a = 0; a < NV; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane / 16) + i;
      float acc = red[(a * kAttnWaves) * 16 + row];
#pragma unroll
      for (int ww = 1; ww < kAttnWaves; ++ww) {
        const float o = red[(a * kAttnWaves + ww) * 16 + row];
        acc = ((MAXMASK >> a) & 1) ? fmaxf(acc, o) : acc + o;
      }
      v[a][i] = acc;
    }
}

// rint(v / s) clamped to [-127, 127], with inv = 1 / s (0 when s = 0)
__device__ __forceinline__ float quant_i8(float v, float inv) {
  return fminf(fmaxf(rintf(v * inv), -127.f), 127.f);
}

// rint(v / s) where |v| <= 127 s by construction (s = max |v| / 127 rounded
// to fp32, inv within an ulp of 1 / s, so |v inv| < 127.5): no clamp
__device__ __forceinline__ float quant_i8_inrange(float v, float inv) { return rintf(v * inv); }

// Everything one chunk of 256 positions needs from the caches: per lane, its
// wave's 4 key tiles and 2 x 2 value tiles, and the per-token scales and
// zero points of its 4 positions.
struct ChunkData {
  u32x4 k[4], v[2][2];
  uint16_t ks[4], kz[4], vs[4], vz[4];
};

// One workgroup per (split, kv head, batch row); a split is `cpw` consecutive
// chunks of 256 positions, walked in order with the next chunk's loads in
// flight while the current one is computed, and merged into a running
// (max, sum, output) per query head (online softmax).  Wave w computes the
// scores of positions 64 w .. 64 w + 63 of each chunk (4 tiles of 16) and the
// outputs of head dimensions 32 w .. 32 w + 31 (2 tiles of 16).
__global__ __launch_bounds__(kAttnThreads) void attn_msd_chunk_kernel(
    const int8_t* __restrict__ qsl, const float* __restrict__ qsc, int MQ, int Hq, int Hkv, int L, int cpw,
    const uint8_t* __restrict__ kp, const uint16_t* __restrict__ ks, const uint16_t* __restrict__ kz,
    const uint8_t* __restrict__ vtp, const uint16_t* __restrict__ vs, const uint16_t* __restrict__ vz,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __align__(16) int8_t psl[2][16][kChunk];  // weight slices in the int8 operand order
  // two reduction buffers, used alternately: four reductions per chunk
  // (max; sum and max; max; sums), so every chunk starts on buffer 0
  __shared__ float red[2][2 * kAttnWaves * 16];

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nsplit = gridDim.x;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ln = lane % 16, kb = lane / 16;
  const size_t bh = (size_t)b * Hkv + h;
  const int qrow0 = b * Hq + h * G;  // first query row of this kv head

  // ---- query operands (rows >= G read as zero) and the output rows' scales
  u32x4 Aq[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int pu = 0; pu < 2; ++pu)
      Aq[j][pu] = ln < G ? *reinterpret_cast<const u32x4*>(qsl + ((size_t)j * MQ + qrow0 + ln) * kHeadDim + 64 * pu + 16 * kb)
                         : u32x4{0, 0, 0, 0};
  float sq[2][4];
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kb + i;
      sq[j][i] = g < G ? qsc[(size_t)j * MQ + qrow0 + g] : 0.f;
    }

  const uint8_t* kbase = kp + bh * (size_t)L * (kHeadDim / 2);
  const uint8_t* vbase = vtp + bh * (size_t)L * (kHeadDim / 2);
  const int ltiles = L / 128;
  // keys (with their scales and zero points) and values are loaded
  // separately: the next chunk's keys go into the registers the current
  // scores are done with, its values into those the current value product is
  // done with, so each load flies while the rest of a chunk is computed
  auto load_keys = [&](int chunk, ChunkData& cd) {
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int tile = chunk * (kChunk / 16) + 4 * w + tt;
      cd.k[tt] = *reinterpret_cast<const u32x4*>(kbase + (size_t)tile * 1024 + 16 * lane);
      const size_t t = bh * L + (size_t)(chunk * kChunk + 64 * w + 16 * tt + ln);
      cd.ks[tt] = ks[t];
      cd.kz[tt] = kz[t];
    }
  };
  auto load_values = [&](int chunk, ChunkData& cd) {
#pragma unroll
    for (int nd = 0; nd < 2; ++nd)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        cd.v[nd][q] =
            *reinterpret_cast<const u32x4*>(vbase + ((size_t)(2 * w + nd) * ltiles + chunk * 2 + q) * 1024 + 16 * lane);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const size_t t = bh * L + (size_t)(chunk * kChunk + 64 * w + 16 * tt + ln);
      cd.vs[tt] = vs[t];
      cd.vz[tt] = vz[t];
    }
  };

  float Mrun[4], Lrun[4], Orun[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Mrun[i] = -INFINITY;
    Lrun[i] = 0.f;
    Orun[0][i] = Orun[1][i] = 0.f;
  }

  ChunkData cur;
  const int c0 = split * cpw;
  load_keys(c0, cur);
  load_values(c0, cur);
  for (int ci = 0; ci < cpw; ++ci) {
    const bool more = ci + 1 < cpw;

    // ---- scores of this wave's 4 token tiles
    float sc[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const float s = half_bits_to_float(cur.ks[tt]);
      const uint32_t zb = (uint32_t)half_bits_to_float(cur.kz[tt]) * 0x01010101u;
      auto qz = [&](uint32_t q) { return ((q | 0x80808080u) - zb) ^ 0x80808080u; };  // bytes q - z
      u32x4 Bk[2];
#pragma unroll
      for (int pu = 0; pu < 2; ++pu) {
        const uint32_t w0 = cur.k[tt][2 * pu], w1 = cur.k[tt][2 * pu + 1];
        Bk[pu] = u32x4{qz(w0 & 0x0F0F0F0Fu), qz((w0 >> 4) & 0x0F0F0F0Fu), qz(w1 & 0x0F0F0F0Fu),
                       qz((w1 >> 4) & 0x0F0F0F0Fu)};
      }
      i32x4 D[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        D[j] = mfma_i8_16x16x64(Aq[j][0], Bk[0], i32x4{0, 0, 0, 0});
        D[j] = mfma_i8_16x16x64(Aq[j][1], Bk[1], D[j]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sc[tt][i] = s * fmaf(sq[0][i], (float)D[0][i], sq[1][i] * (float)D[1][i]) * kScoreScale;
    }

    if (more) load_keys(c0 + ci + 1, cur);  // in flight during the rest of this chunk

    // ---- chunk softmax: max, then p = exp(score - max); its sum and the
    // max of the weights w = p sV (w >= 0) in one reduction
    float m[1][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) m[0][i] = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
    reduce_rows<1, 1>(m, red[0], w, lane);
    float sv[4];
    int zv[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      sv[tt] = half_bits_to_float(cur.vs[tt]);
      zv[tt] = (int)half_bits_to_float(cur.vz[tt]);
    }
    float p[4][4], la[2][4];  // la[0]: row sum of exp, la[1]: row max of the weights
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      la[0][i] = 0.f;
      la[1][i] = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float e = __builtin_amdgcn_exp2f(sc[tt][i] - m[0][i]);
        la[0][i] += e;
        p[tt][i] = e * sv[tt];
        la[1][i] = fmaxf(la[1][i], p[tt][i]);
      }
    }
    reduce_rows<2, 2>(la, red[1], w, lane);
    float(&l)[4] = la[0];
    float(&amax)[4] = la[1];

    // ---- the weights split into two int8 slices per row
    float r1[4], r2[4], amax2[1][4];
    int A1[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r1[i] = amax[i] * (1.f / 127.f);
      const float inv = r1[i] > 0.f ? 1.f / r1[i] : 0.f;
      amax2[0][i] = 0.f;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const float a = quant_i8(p[tt][i], inv);
        A1[tt][i] = (int)a;
        p[tt][i] = p[tt][i] - r1[i] * a;  // residual
        amax2[0][i] = fmaxf(amax2[0][i], fabsf(p[tt][i]));
      }
    }
    reduce_rows<1, 1>(amax2, red[0], w, lane);
    float zt[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r2[i] = amax2[0][i] * (1.f / 127.f);
      const float inv = r2[i] > 0.f ? 1.f / r2[i] : 0.f;
      int z0 = 0, z1 = 0;
      const int row = 4 * kb + i;
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        const int a2 = (int)quant_i8(p[tt][i], inv);
        z0 += A1[tt][i] * zv[tt];
        z1 += a2 * zv[tt];
        // position tc of the chunk in the int8 operand order: per 64 positions,
        // 64 b + 32 hh + 8 k + e sits at byte 64 b + 16 k + 8 hh + p(e),
        // p(0..7) = 0, 2, 4, 6, 1, 3, 5, 7
        const int tc = 64 * w + 16 * tt + ln;
        const int bb = tc / 64, pos = tc % 64, hh = pos / 32, kk = (pos % 32) / 8, e = pos % 8;
        const int byte = 64 * bb + 16 * kk + 8 * hh + (e < 4 ? 2 * e : 2 * (e - 4) + 1);
        psl[0][row][byte] = (int8_t)A1[tt][i];
        psl[1][row][byte] = (int8_t)a2;
      }
      zt[0][i] = (float)z0;  // |sum| <= 256 * 127 * 15 < 2^24: exact
      zt[1][i] = (float)z1;
    }
    reduce_rows<0, 2>(zt, red[1], w, lane);  // its barrier also publishes psl

    // ---- values: this wave's 2 tiles of 16 head dimensions, merged into the
    // running output (the next chunk writes psl only after its first barrier,
    // which every wave reaches after these reads)
    float fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float mn = fmaxf(Mrun[i], m[0][i]);
      fa[i] = __builtin_amdgcn_exp2f(Mrun[i] - mn);
      fb[i] = __builtin_amdgcn_exp2f(m[0][i] - mn);
      Lrun[i] = fmaf(fa[i], Lrun[i], fb[i] * l[i]);
      Mrun[i] = mn;
    }
#pragma unroll
    for (int nd = 0; nd < 2; ++nd) {
      i32x4 E[2] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t w0 = cur.v[nd][u / 2][2 * (u % 2)], w1 = cur.v[nd][u / 2][2 * (u % 2) + 1];
        const u32x4 Bv{w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const u32x4 Ap = *reinterpret_cast<const u32x4*>(&psl[j][ln][64 * u + 16 * kb]);
          E[j] = mfma_i8_16x16x64(Ap, Bv, E[j]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float o = fmaf(r1[i], (float)E[0][i] - zt[0][i], r2[i] * ((float)E[1][i] - zt[1][i]));
        Orun[nd][i] = fmaf(fa[i], Orun[nd][i], fb[i] * o);
      }
    }
    if (more) load_values(c0 + ci + 1, cur);
  }

#pragma unroll
  for (int nd = 0; nd < 2; ++nd)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kb + i;
      if (g < G) part_o[(((size_t)(qrow0 + g)) * nsplit + split) * kHeadDim + 16 * (2 * w + nd) + ln] = Orun[nd][i];
    }
  if (w == 0 && ln == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kb + i;
      if (g < G) {
        part_ml[(((size_t)(qrow0 + g)) * nsplit + split) * 2] = Mrun[i];
        part_ml[(((size_t)(qrow0 + g)) * nsplit + split) * 2 + 1] = Lrun[i];
      }
    }
}

// ---------------------------------------------------------------------------
// One wave per chunk (G <= 8 query heads per key/value head).  With at most 8
// heads, the 16 rows of a product hold both slices at once: rows 0-7 the
// first slice of heads 0-7, rows 8-15 the second, so one pair of products
// gives both D_1 and D_2 of a key tile.  The results of two tiles A and B are
// then exchanged between the lane halves (v_permlane32_swap: lanes 32-63 of
// the first with lanes 0-31 of the second), after which lane l holds, for
// heads 4 hq + i (hq = (l / 16) mod 2), D_1 and D_2 of token l mod 16 of tile
// A (l < 32) or B (l >= 32): every lane carries useful values, and the
// softmax and slicing work per lane is half that of a 16-head layout.  The
// value product stacks the weight slices the same way.  A wave's row
// reductions stay inside the wave (DPP within 16 lanes, then the two halves),
// so no workgroup barrier is needed per chunk; the 4 waves of a workgroup
// (4 consecutive chunks) merge their (max, sum, output) once at the end.
__device__ __forceinline__ void swap_halves(int& a, int& b) {
  const auto r = __builtin_amdgcn_permlane32_swap((unsigned)a, (unsigned)b, false, false);
  a = (int)r[0];
  b = (int)r[1];
}

// reduction over the 32 lanes that hold the same heads: the 16 lanes of a
// row group, then lane l with lane l ^ 32
template <RowOp OP>
__device__ __forceinline__ float row32(float v) {
  v = row16<OP>(v);
  int a = __builtin_bit_cast(int, v), b = a;
  swap_halves(a, b);  // a: lanes 0-31 of v on both halves, b: lanes 32-63
  if constexpr (OP == kRowMaxNonNeg) return __builtin_bit_cast(float, max((uint32_t)a, (uint32_t)b));
  const float x = __builtin_bit_cast(float, a), y = __builtin_bit_cast(float, b);
  return OP == kRowMax ? fmaxf(x, y) : x + y;
}

// byte offset of chunk position t in the int8 operand order: per 64
// positions, 64 b + 32 hh + 8 k + e sits at byte 64 b + 16 k + 8 hh + p(e),
// p(0..7) = 0, 2, 4, 6, 1, 3, 5, 7
__device__ __forceinline__ int operand_byte(int t) {
  const int bb = t / 64, pos = t % 64, hh = pos / 32, kk = (pos % 32) / 8, e = pos % 8;
  return 64 * bb + 16 * kk + 8 * hh + (e < 4 ? 2 * e : 2 * (e - 4) + 1);
}

__global__ __launch_bounds__(kAttnThreads) void attn_msd_wave_kernel(
    const uint16_t* __restrict__ qh, int MQ, int Hq, int Hkv, int L,
    const uint8_t* __restrict__ kp, const uint16_t* __restrict__ ks, const uint16_t* __restrict__ kz,
    const uint8_t* __restrict__ vtp, const uint16_t* __restrict__ vs, const uint16_t* __restrict__ vz,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __align__(16) int8_t psl[kAttnWaves][16][kChunk];  // each wave's stacked weight slices
  __shared__ float mo[kAttnWaves][8][kHeadDim];                  // each wave's chunk output
  __shared__ float mml[kAttnWaves][8][2];                        // and its (max, sum) per head

  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nsplit = gridDim.x;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ln = lane % 16, kb = lane / 16;
  const int hi = lane / 32, hq = kb % 2;  // after the swaps: tile half, head quad
  const size_t bh = (size_t)b * Hkv + h;
  const int qrow0 = b * Hq + h * G;
  const int chunk = split * kAttnWaves + w;
  const int ltiles = L / 128;

  float Mw[4], Lw[4], O[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    Mw[i] = -INFINITY;
    Lw[i] = 0.f;
#pragma unroll
    for (int np = 0; np < 4; ++np) O[np][i] = 0.f;
  }

  const bool has_chunk = chunk < L / kChunk;  // wave-uniform
  const size_t tok0 = bh * L + (size_t)chunk * kChunk;
  // Vector loads return in the order they were issued (per wave, and
  // through the CU's memory pipeline), so a wait also waits for the loads
  // issued before: the loads go out in the order of first use.  First the
  // queries the split below needs, then the key scales and zero points and
  // the chunk's 16 key tiles (the scores need both); the value side below
  // likewise.
  const int gh = 2 * w + lane / 32, d0 = 4 * (lane % 32);  // this lane's head and dimensions in the split
  u32x2 xq = {0, 0};
  if (gh < G) xq = *reinterpret_cast<const u32x2*>(qh + (size_t)(qrow0 + gh) * kHeadDim + d0);
  // the scales and zero points of the tokens the lane holds after the swaps
  // (token ln of tile 2 p + hi), each in a register of its own (two in one
  // register would make the wave wait for them here), and the 16 key tiles.
  // A wave without a chunk (at the end of a row whose chunk count is not a
  // multiple of 4) loads chunk 0 instead and ignores it: no branch between
  // these loads and the split, which would make the split wait for them all.
  const size_t ktok0 = has_chunk ? tok0 : bh * L;
  uint32_t zk[8], sk[8];
  u32x4 T[16];
#pragma unroll
  for (int pp = 0; pp < 8; ++pp) {
    zk[pp] = kz[ktok0 + 16 * (2 * pp + hi) + ln];
    sk[pp] = ks[ktok0 + 16 * (2 * pp + hi) + ln];
  }
  const uint8_t* kbase = kp + (bh * (size_t)(L / 16) + (size_t)(has_chunk ? chunk : 0) * 16) * 1024 + 16 * lane;
#pragma unroll
  for (int t = 0; t < 16; ++t) T[t] = *reinterpret_cast<const u32x4*>(kbase + (size_t)t * 1024);
  __builtin_amdgcn_sched_barrier(0);  // the key loads go out before the split

  // ---- the group's queries split into two int8 slices with the decisions
  // of the decomposition kernel, taken in fp32 (per head: s_1 = fp32(max|q| /
  // 127), A_1 = rint(q / s_1), r = q - s_1 A_1, s_2 = fp32(max|r| / 127),
  // A_2 = rint(r / s_2)), while the key loads are in flight.  The workgroup's
  // four waves share one split: wave w takes heads 2 w and 2 w + 1, 32 lanes
  // per head and 4 dimensions per lane, and the codes go to qop (slice 1 of
  // head g in row g, slice 2 in row 8 + g, operand order), from which every
  // wave reads its stacked A operands: row ln = slice ln / 8 of head ln mod 8.
  __shared__ __align__(16) int8_t qop[16][kHeadDim];
  __shared__ float qscale[2][8];
  {
    float xf[4];
    uint32_t mag = 0;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      xf[2 * i] = half_bits_to_float((uint16_t)(xq[i] & 0xFFFFu));
      xf[2 * i + 1] = half_bits_to_float((uint16_t)(xq[i] >> 16));
      const uint32_t m2 = xq[i] & 0x7FFF7FFFu;  // magnitude bits order like the magnitudes
      mag = max(mag, max(m2 & 0xFFFFu, m2 >> 16));
    }
    auto max32 = [](uint32_t v) {  // over the 32 lanes of a head
#pragma unroll
      for (int off = 1; off < 32; off <<= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, kWave));
      return v;
    };
    auto store4 = [&](int row, const float (&q)[4]) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qop[row][operand_byte(d0 + e)] = (int8_t)(int)q[e];  // in [-127, 127] without a clamp
    };
    mag = max32(mag);
    const double s1 = (double)(float)((double)half_bits_to_float((uint16_t)mag) / 127.0);
    const float s1f = (float)s1, inv1 = s1 != 0.0 ? (float)(1.0 / s1) : 0.f;
    float q[4];
    float dmax = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = rint127_fast(xf[e], inv1, dmax);
    if (near127(dmax)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = decide127((double)xf[e], s1, inv1);
    }
    store4(gh, q);  // a head beyond G has x = 0: zero codes and scales
    // r = x - s_1 A_1 is exact in fp32.  For A_1 = 0 it is x.  Otherwise
    // |x| >= s_1 / 2, so x is a multiple of s_1's ulp (the fp16 grid at |x|
    // is at least 2^12 of them), and |r| <= s_1 / 2 is at most 2^23 of them.
    float rf[4];
    uint32_t mag2 = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rf[e] = fmaf(-s1f, q[e], xf[e]);
      mag2 = max(mag2, __float_as_uint(fabsf(rf[e])));
    }
    mag2 = max32(mag2);
    const double s2 = (double)(float)((double)__uint_as_float(mag2) / 127.0);
    const float inv2 = s2 != 0.0 ? (float)(1.0 / s2) : 0.f;
    dmax = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) q[e] = rint127_fast(rf[e], inv2, dmax);
    if (near127(dmax)) {
#pragma unroll
      for (int e = 0; e < 4; ++e) q[e] = decide127((double)rf[e], s2, inv2);
    }
    store4(8 + gh, q);
    if (lane % 32 == 0) {
      qscale[0][gh] = (float)s1;
      qscale[1][gh] = (float)s2;
    }
  }
  __syncthreads();

  int8_t* my = &psl[w][0][0];
  if (has_chunk) {
    // ---- the chunk's 16 value tiles (V^T: 8 tiles of 16 dimensions by 2 of
    // 128 positions), issued once the decomposition's registers are free;
    // they fly during the scores and the softmax.  Their scales and zero
    // points go first: the softmax and the weight slicing need them.
    uint16_t sv16[8], zv16[8];
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      sv16[pp] = vs[tok0 + 16 * (2 * pp + hi) + ln];
      zv16[pp] = vz[tok0 + 16 * (2 * pp + hi) + ln];
    }
    u32x4 V[16];
    const uint8_t* vbase = vtp + bh * (size_t)L * (kHeadDim / 2) + 16 * lane;
#pragma unroll
    for (int nd = 0; nd < 8; ++nd)
#pragma unroll
      for (int q = 0; q < 2; ++q)
        V[2 * nd + q] = *reinterpret_cast<const u32x4*>(vbase + ((size_t)nd * ltiles + chunk * 2 + q) * 1024);
    __builtin_amdgcn_sched_barrier(0);  // all value loads go out before the first wait for the keys

    u32x4 Aq[2];
#pragma unroll
    for (int pu = 0; pu < 2; ++pu) Aq[pu] = *reinterpret_cast<const u32x4*>(&qop[ln][64 * pu + 16 * kb]);
    float s1q[4], s2q[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s1q[i] = qscale[0][4 * hq + i];
      s2q[i] = qscale[1][4 * hq + i];
    }
    // the key zero point enters after the product: D_j = sum_d A_j q - zK
    // sum_d A_j, with the row sums of the query slices from one product
    // against ones (exact: every term is an integer below 2^24)
    float sA1[4], sA2[4];
    {
      const u32x4 ones{0x01010101u, 0x01010101u, 0x01010101u, 0x01010101u};
      i32x4 S = mfma_i8_16x16x64(Aq[0], ones, i32x4{0, 0, 0, 0});
      S = mfma_i8_16x16x64(Aq[1], ones, S);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int x = S[i], y = S[i];
        swap_halves(x, y);
        sA1[i] = (float)x;
        sA2[i] = (float)y;
      }
    }

    // ---- scores: tile pairs (2 p, 2 p + 1)
      float sc[8][4];
#pragma unroll
    for (int pp = 0; pp < 8; ++pp) {
      i32x4 D[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4& kt = T[2 * pp + hh];
        u32x4 Bk[2];
#pragma unroll
        for (int pu = 0; pu < 2; ++pu) {
          const uint32_t w0 = kt[2 * pu], w1 = kt[2 * pu + 1];
          Bk[pu] = u32x4{w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
        }
        D[hh] = mfma_i8_16x16x64(Aq[0], Bk[0], i32x4{0, 0, 0, 0});
        D[hh] = mfma_i8_16x16x64(Aq[1], Bk[1], D[hh]);
      }
      const float skf = half_bits_to_float((uint16_t)sk[pp]) * kScoreScale;
      const float zkf = half_bits_to_float((uint16_t)zk[pp]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int x = D[0][i], y = D[1][i];
        swap_halves(x, y);  // x: D_1, y: D_2 of token ln of tile 2 pp + hi, head 4 hq + i (before zK)
        const float d1 = fmaf(-zkf, sA1[i], (float)x), d2 = fmaf(-zkf, sA2[i], (float)y);
        sc[pp][i] = skf * fmaf(s1q[i], d1, s2q[i] * d2);
      }
    }

    // ---- softmax over the chunk, weights w = p sV, their two int8 slices
    float m[4], l[4], am[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m[i] = sc[0][i];
#pragma unroll
      for (int pp = 1; pp < 8; ++pp) m[i] = fmaxf(m[i], sc[pp][i]);
      m[i] = row32<kRowMax>(m[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      l[i] = 0.f;
      am[i] = 0.f;
#pragma unroll
      for (int pp = 0; pp < 8; ++pp) {
        const float e = __builtin_amdgcn_exp2f(sc[pp][i] - m[i]);
        l[i] += e;
        sc[pp][i] = e * half_bits_to_float(sv16[pp]);
        am[i] = fmaxf(am[i], sc[pp][i]);
      }
      l[i] = row32<kRowSum>(l[i]);
      am[i] = row32<kRowMaxNonNeg>(am[i]);  // w = p sV >= 0
    }
    float r1[4], r2[4], zt1[4], zt2[4];  // the weight slices go to this wave's LDS rows
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r1[i] = am[i] * (1.f / 127.f);
      const float inv1 = r1[i] > 0.f ? __builtin_amdgcn_rcpf(r1[i]) : 0.f;  // 1 ulp: the codes are compared within a tolerance
      float am2 = 0.f, z1 = 0.f;  // integer sums below 2^24: exact in fp32
#pragma unroll
      for (int pp = 0; pp < 8; ++pp) {
        const float a = quant_i8_inrange(sc[pp][i], inv1);
        const int t = 16 * (2 * pp + hi) + ln;
        my[(4 * hq + i) * kChunk + operand_byte(t)] = (int8_t)(int)a;
        z1 = fmaf(a, half_bits_to_float(zv16[pp]), z1);
        sc[pp][i] = sc[pp][i] - r1[i] * a;
        am2 = fmaxf(am2, fabsf(sc[pp][i]));
      }
      r2[i] = row32<kRowMaxNonNeg>(am2) * (1.f / 127.f);
      const float inv2 = r2[i] > 0.f ? __builtin_amdgcn_rcpf(r2[i]) : 0.f;
      float z2 = 0.f;
#pragma unroll
      for (int pp = 0; pp < 8; ++pp) {
        const float a = quant_i8_inrange(sc[pp][i], inv2);
        const int t = 16 * (2 * pp + hi) + ln;
        my[(8 + 4 * hq + i) * kChunk + operand_byte(t)] = (int8_t)(int)a;
        z2 = fmaf(a, half_bits_to_float(zv16[pp]), z2);
      }
      zt1[i] = row32<kRowSum>(z1);  // |sum| <= 256 * 127 * 15 < 2^24: exact
      zt2[i] = row32<kRowSum>(z2);
    }

    // ---- values: E (rows 0-7 slice 1, 8-15 slice 2) per dim tile, pairs of
    // dim tiles exchanged between the halves like the scores.  The slices
    // were written by this wave; its LDS accesses complete in order.
    u32x4 Av[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) Av[u] = *reinterpret_cast<const u32x4*>(my + ln * kChunk + 64 * u + 16 * kb);
#pragma unroll
    for (int np = 0; np < 4; ++np) {
      i32x4 E[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int nd = 2 * np + hh;
        E[hh] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const u32x4& vt = V[2 * nd + u / 2];
          const uint32_t w0 = vt[2 * (u % 2)], w1 = vt[2 * (u % 2) + 1];
          const u32x4 Bv{w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
          E[hh] = mfma_i8_16x16x64(Av[u], Bv, E[hh]);
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        int x = E[0][i], y = E[1][i];
        swap_halves(x, y);  // dim 16 (2 np + hi) + ln, head 4 hq + i
        O[np][i] = fmaf(r1[i], (float)x - zt1[i], r2[i] * ((float)y - zt2[i]));
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      Mw[i] = m[i];
      Lw[i] = l[i];
    }
  }

  // ---- merge the workgroup's chunks: (max, sum) and the unnormalised output
  // relative to the merged max, as one partial of this split
  if (ln == 0 && hi == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mml[w][4 * hq + i][0] = Mw[i];
      mml[w][4 * hq + i][1] = Lw[i];
    }
#pragma unroll
  for (int np = 0; np < 4; ++np)
#pragma unroll
    for (int i = 0; i < 4; ++i) mo[w][4 * hq + i][16 * (2 * np + hi) + ln] = O[np][i];
  __syncthreads();
  for (int e = tid; e < 8 * kHeadDim; e += kAttnThreads) {
    const int g = e / kHeadDim, n = e % kHeadDim;
    if (g >= G) break;  // e grows with g
    float mx = mml[0][g][0];
#pragma unroll
    for (int ww = 1; ww < kAttnWaves; ++ww) mx = fmaxf(mx, mml[ww][g][0]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int ww = 0; ww < kAttnWaves; ++ww) {
      const float f = __builtin_amdgcn_exp2f(mml[ww][g][0] - mx);  // 0 for a wave without a chunk
      num = fmaf(f, mo[ww][g][n], num);
      den = fmaf(f, mml[ww][g][1], den);
    }
    const size_t row = (size_t)(qrow0 + g) * nsplit + split;
    part_o[row * kHeadDim + n] = num;
    if (n == 0) {
      part_ml[row * 2] = mx;
      part_ml[row * 2 + 1] = den;
    }
  }
}

// one workgroup of 128 threads per query row: o[n] = sum_s e^(m_s - m) o_s[n]
// / sum_s e^(m_s - m) l_s over the splits, in order.  Every thread loads the
// splits' (max, sum) pairs and its outputs eight splits at a time, all of a
// batch's loads issued before any is used (one memory round trip per eight
// splits).
__global__ __launch_bounds__(kHeadDim) void attn_combine_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_ml, int nsplit,
                                                                uint16_t* __restrict__ out) {
  const size_t row = blockIdx.x;
  const int n = threadIdx.x;
  const float2* ml = reinterpret_cast<const float2*>(part_ml) + row * nsplit;
  const float* po = part_o + row * nsplit * kHeadDim + n;
  float m = -INFINITY, num = 0.f, den = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += 8) {
    float2 v[8];
    float o[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = c0 + i < nsplit ? ml[c0 + i] : make_float2(-INFINITY, 0.f);
      o[i] = c0 + i < nsplit ? po[(size_t)(c0 + i) * kHeadDim] : 0.f;
    }
    float mb = m;
#pragma unroll
    for (int i = 0; i < 8; ++i) mb = fmaxf(mb, v[i].x);
    const float f0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mb);  // rescale what came before
    num *= f0;
    den *= f0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float f = v[i].x == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(v[i].x - mb);
      num = fmaf(f, o[i], num);
      den = fmaf(f, v[i].y, den);
    }
    m = mb;
  }
  out[row * kHeadDim + n] = float_to_half_bits(num / den);
}

}  // namespace

// chunks of 256 positions per workgroup: double while the grid keeps at least
// 512 workgroups (2 per CU, the occupancy of the chunk kernel) and the count
// divides the chunks (at batch 8, 64/8 heads, L = 8192: 1, 2, 4, 8 chunks take
// 44, 40, 38, 45 us).  W4_ATTN_CPW overrides it.
int attn_chunks_per_split(int B, int Hkv, int L) {
  const int nchunk = L / kChunk;
  const char* e = std::getenv("W4_ATTN_CPW");
  int cpw = 1;
  if (e && *e) {
    cpw = std::atoi(e);
    if (cpw < 1 || nchunk % cpw) cpw = 1;
  } else {
    while (nchunk % (2 * cpw) == 0 && (long)(nchunk / (2 * cpw)) * Hkv * B >= 512) cpw *= 2;
  }
  return cpw;
}

// W4_ATTN_WAVE=0 selects the chunk-split kernel for every G (comparison runs).
bool attn_wave_kernel_enabled() {
  const char* e = std::getenv("W4_ATTN_WAVE");
  return !(e && *e == '0');
}

size_t attn_workspace_bytes(int B, int Hq, int L) {
  const size_t MQ = (size_t)B * Hq;
  const size_t nchunk = (size_t)L / kChunk;
  const size_t sl = (2 * MQ * kHeadDim + 255) / 256 * 256;
  const size_t sc = (2 * MQ * sizeof(float) + 255) / 256 * 256;
  const size_t po = (MQ * nchunk * kHeadDim * sizeof(float) + 255) / 256 * 256;
  const size_t pm = (MQ * nchunk * 2 * sizeof(float) + 255) / 256 * 256;
  return sl + sc + po + pm;
}

int launch_attn_msd(const uint16_t* q, int B, int Hq, int Hkv, int L, const uint8_t* kp, const uint16_t* ks,
                    const uint16_t* kz, const uint8_t* vtp, const uint16_t* vs, const uint16_t* vz, uint16_t* out,
                    void* ws, hipStream_t s) {
  const int MQ = B * Hq;
  const int nchunk = L / kChunk;
  char* base = static_cast<char*>(ws);
  int8_t* qsl = reinterpret_cast<int8_t*>(base);
  base += (2 * (size_t)MQ * kHeadDim + 255) / 256 * 256;
  float* qsc = reinterpret_cast<float*>(base);
  base += (2 * (size_t)MQ * sizeof(float) + 255) / 256 * 256;
  float* po = reinterpret_cast<float*>(base);
  base += ((size_t)MQ * nchunk * kHeadDim * sizeof(float) + 255) / 256 * 256;
  float* pm = reinterpret_cast<float*>(base);
  int nsplit, st;
  if (Hq / Hkv <= 8 && attn_wave_kernel_enabled()) {
    nsplit = (nchunk + kAttnWaves - 1) / kAttnWaves;
    hipLaunchKernelGGL(attn_msd_wave_kernel, dim3(nsplit, Hkv, B), dim3(kAttnThreads), 0, s, q, MQ, Hq, Hkv, L, kp,
                       ks, kz, vtp, vs, vz, po, pm);
    st = check_launch("attn_msd_wave");
  } else {
    st = launch_decompose(q, MQ, kHeadDim, 2, false, qsl, nullptr, qsc, s);
    if (st != 0) return st;
    const int cpw = attn_chunks_per_split(B, Hkv, L);
    nsplit = nchunk / cpw;
    hipLaunchKernelGGL(attn_msd_chunk_kernel, dim3(nsplit, Hkv, B), dim3(kAttnThreads), 0, s, qsl, qsc, MQ, Hq, Hkv,
                       L, cpw, kp, ks, kz, vtp, vs, vz, po, pm);
    st = check_launch("attn_msd_chunk");
  }
  if (st != 0) return st;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(MQ), dim3(kHeadDim), 0, s, po, pm, nsplit, out);
  return check_launch("attn_combine");
}

}  // namespace w4

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

__device__ __forceinline__ i32x4 mfma_i8_16x16x64(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// all-reduce over the 16 lanes of a DPP row (the lanes holding one row group
// of a matrix-core output): swap within pairs and quads, then the row's
// half-mirror (lane i with 7 - i) and mirror (lane i with 15 - i)
template <bool MAX>
__device__ __forceinline__ float row16(float v) {
  auto step = [](float x, int ctrl) {
    int y;
    switch (ctrl) {  // the control must be a constant
      case 0:
        y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
        break;
      case 1:
        y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
        break;
      case 2:
        y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false);  // half mirror
        break;
      default:
        y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false);  // mirror
    }
    return __builtin_bit_cast(float, y);
  };
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const float o = step(v, c);
    v = MAX ? fmaxf(v, o) : v + o;
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
    for (int i = 0; i < 4; ++i) v[a][i] = ((MAXMASK >> a) & 1) ? row16<true>(v[a][i]) : row16<false>(v[a][i]);
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

  const float inv_sqrt_d = 0.08838834764831845f;  // 1 / sqrt(128)
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
        sc[tt][i] = s * fmaf(sq[0][i], (float)D[0][i], sq[1][i] * (float)D[1][i]) * inv_sqrt_d;
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
        const float e = __expf(sc[tt][i] - m[0][i]);
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
      fa[i] = __expf(Mrun[i] - mn);
      fb[i] = __expf(m[0][i] - mn);
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

// one workgroup of 128 threads per query row: o[n] = sum_s e^(m_s - m) o_s[n]
// / sum_s e^(m_s - m) l_s over the splits, in order (every thread reads the
// splits' maxima and sums; the outputs eight splits at a time)
__global__ __launch_bounds__(kHeadDim) void attn_combine_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_ml, int nsplit,
                                                                uint16_t* __restrict__ out) {
  const size_t row = blockIdx.x;
  const int n = threadIdx.x;
  const float* ml = part_ml + row * nsplit * 2;
  float m = -INFINITY;
  for (int c = 0; c < nsplit; ++c) m = fmaxf(m, ml[2 * c]);
  float num = 0.f, den = 0.f;
  const float* po = part_o + row * nsplit * kHeadDim + n;
  for (int c0 = 0; c0 < nsplit; c0 += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = c0 + i < nsplit ? po[(size_t)(c0 + i) * kHeadDim] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (c0 + i < nsplit) {
        const float f = expf(ml[2 * (c0 + i)] - m);
        num = fmaf(f, v[i], num);
        den = fmaf(f, ml[2 * (c0 + i) + 1], den);
      }
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
  int st = launch_decompose(q, MQ, kHeadDim, 2, false, qsl, nullptr, qsc, s);
  if (st != 0) return st;
  const int cpw = attn_chunks_per_split(B, Hkv, L);
  const int nsplit = nchunk / cpw;
  hipLaunchKernelGGL(attn_msd_chunk_kernel, dim3(nsplit, Hkv, B), dim3(kAttnThreads), 0, s, qsl, qsc, MQ, Hq, Hkv, L,
                     cpw, kp, ks, kz, vtp, vs, vz, po, pm);
  st = check_launch("attn_msd_chunk");
  if (st != 0) return st;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(MQ), dim3(kHeadDim), 0, s, po, pm, nsplit, out);
  return check_launch("attn_combine");
}

}  // namespace w4

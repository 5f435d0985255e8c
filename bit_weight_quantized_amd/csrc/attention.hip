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

namespace w4 {
namespace {

constexpr int kHeadDim = 128;
constexpr int kChunk = 256;
constexpr int kAttnThreads = 256;  // 4 waves
constexpr int kAttnWaves = kAttnThreads / kWave;

__device__ __forceinline__ i32x4 mfma_i8_16x16x64(u32x4 a, u32x4 b, i32x4 c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, a), __builtin_bit_cast(i32x4, b), c, 0, 0, 0);
}

// sum / max over the 16 lanes of a 16-lane group (the lanes holding one row
// group of an MFMA output), then over the waves through LDS; every lane
// returns the totals of its 4 rows (4 kb + i)
template <bool MAX, typename T>
__device__ __forceinline__ void reduce_rows(T (&v)[4], T* red, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const T o = __shfl_xor(v[i], off);
      v[i] = MAX ? (v[i] > o ? v[i] : o) : v[i] + o;
    }
  __syncthreads();  // red is free
  if (lane % 16 == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w * 16 + 4 * (lane / 16) + i] = v[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (lane / 16) + i;
    T acc = red[row];
#pragma unroll
    for (int ww = 1; ww < kAttnWaves; ++ww) {
      const T o = red[ww * 16 + row];
      acc = MAX ? (acc > o ? acc : o) : acc + o;
    }
    v[i] = acc;
  }
}

__device__ __forceinline__ float quant_i8(float v, float s) {
  return s != 0.f ? fminf(fmaxf(rintf(v / s), -127.f), 127.f) : 0.f;
}

// One workgroup per (chunk, kv head, batch row).  Wave w computes the scores
// of tokens 64 w .. 64 w + 63 of the chunk (4 tiles of 16) and the outputs of
// head dimensions 32 w .. 32 w + 31 (2 tiles of 16).
__global__ __launch_bounds__(kAttnThreads) void attn_msd_chunk_kernel(
    const int8_t* __restrict__ qsl, const float* __restrict__ qsc, int MQ, int Hq, int Hkv, int L,
    const uint8_t* __restrict__ kp, const uint16_t* __restrict__ ks, const uint16_t* __restrict__ kz,
    const uint8_t* __restrict__ vtp, const uint16_t* __restrict__ vs, const uint16_t* __restrict__ vz,
    float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ __align__(16) int8_t psl[2][16][kChunk];  // weight slices in the int8 operand order
  __shared__ float redf[kAttnWaves * 16];
  __shared__ int redi[kAttnWaves * 16];

  const int chunk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int nchunk = gridDim.x;
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

  // ---- scores of this wave's 4 token tiles
  const uint8_t* kbase = kp + bh * (size_t)L * (kHeadDim / 2);
  const float inv_sqrt_d = 0.08838834764831845f;  // 1 / sqrt(128)
  float sc[4][4];
  int tok[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int tile = chunk * (kChunk / 16) + 4 * w + tt;
    const int t = 16 * tile + ln;
    tok[tt] = t;
    const u32x4 Kw = *reinterpret_cast<const u32x4*>(kbase + (size_t)tile * 1024 + 16 * lane);
    const float s = half_bits_to_float(ks[bh * L + t]);
    const uint32_t zb = (uint32_t)half_bits_to_float(kz[bh * L + t]) * 0x01010101u;
    auto qz = [&](uint32_t q) { return ((q | 0x80808080u) - zb) ^ 0x80808080u; };  // bytes q - z
    u32x4 Bk[2];
#pragma unroll
    for (int pu = 0; pu < 2; ++pu) {
      const uint32_t w0 = Kw[2 * pu], w1 = Kw[2 * pu + 1];
      Bk[pu] = u32x4{qz(w0 & 0x0F0F0F0Fu), qz((w0 >> 4) & 0x0F0F0F0Fu), qz(w1 & 0x0F0F0F0Fu), qz((w1 >> 4) & 0x0F0F0F0Fu)};
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

  // ---- chunk softmax: max, then p = exp(score - max) and its sum
  float m[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) m[i] = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
  reduce_rows<true>(m, redf, w, lane);
  float p[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    l[i] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      p[tt][i] = expf(sc[tt][i] - m[i]);
      l[i] += p[tt][i];
    }
  }
  reduce_rows<false>(l, redf, w, lane);

  // ---- weights times the value scale, split into two int8 slices per row
  float sv[4];
  int zv[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    sv[tt] = half_bits_to_float(vs[bh * L + tok[tt]]);
    zv[tt] = (int)half_bits_to_float(vz[bh * L + tok[tt]]);
  }
  float amax[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    amax[i] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      p[tt][i] *= sv[tt];  // w = p sV >= 0
      amax[i] = fmaxf(amax[i], p[tt][i]);
    }
  }
  reduce_rows<true>(amax, redf, w, lane);
  float r1[4], r2[4], amax2[4];
  int A1[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r1[i] = amax[i] / 127.f;
    amax2[i] = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const float a = quant_i8(p[tt][i], r1[i]);
      A1[tt][i] = (int)a;
      p[tt][i] = p[tt][i] - r1[i] * a;  // residual
      amax2[i] = fmaxf(amax2[i], fabsf(p[tt][i]));
    }
  }
  reduce_rows<true>(amax2, redf, w, lane);
  int zt[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    r2[i] = amax2[i] / 127.f;
    zt[0][i] = zt[1][i] = 0;
    const int row = 4 * kb + i;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int a2 = (int)quant_i8(p[tt][i], r2[i]);
      zt[0][i] += A1[tt][i] * zv[tt];
      zt[1][i] += a2 * zv[tt];
      // position tc of the chunk in the int8 operand order: per 64 positions,
      // 64 b + 32 hh + 8 k + e sits at byte 64 b + 16 k + 8 hh + p(e),
      // p(0..7) = 0, 2, 4, 6, 1, 3, 5, 7
      const int tc = 64 * w + 16 * tt + ln;
      const int bb = tc / 64, pos = tc % 64, hh = pos / 32, kk = (pos % 32) / 8, e = pos % 8;
      const int byte = 64 * bb + 16 * kk + 8 * hh + (e < 4 ? 2 * e : 2 * (e - 4) + 1);
      psl[0][row][byte] = (int8_t)A1[tt][i];
      psl[1][row][byte] = (int8_t)a2;
    }
  }
  reduce_rows<false>(zt[0], redi, w, lane);
  reduce_rows<false>(zt[1], redi, w, lane);  // also publishes psl (barriers inside)

  // ---- values: this wave's 2 tiles of 16 head dimensions
  const uint8_t* vbase = vtp + bh * (size_t)L * (kHeadDim / 2);
  const int ltiles = L / 128;
#pragma unroll
  for (int nd = 0; nd < 2; ++nd) {
    const int dt = 2 * w + nd;  // d rows 16 dt .. 16 dt + 15
    u32x4 Vw[2];
#pragma unroll
    for (int q = 0; q < 2; ++q)
      Vw[q] = *reinterpret_cast<const u32x4*>(vbase + ((size_t)dt * ltiles + chunk * 2 + q) * 1024 + 16 * lane);
    i32x4 E[2] = {i32x4{0, 0, 0, 0}, i32x4{0, 0, 0, 0}};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w0 = Vw[u / 2][2 * (u % 2)], w1 = Vw[u / 2][2 * (u % 2) + 1];
      const u32x4 Bv{w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const u32x4 Ap = *reinterpret_cast<const u32x4*>(&psl[j][ln][64 * u + 16 * kb]);
        E[j] = mfma_i8_16x16x64(Ap, Bv, E[j]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kb + i;
      if (g >= G) continue;
      const float o = fmaf(r1[i], (float)(E[0][i] - zt[0][i]), r2[i] * (float)(E[1][i] - zt[1][i]));
      part_o[(((size_t)(qrow0 + g)) * nchunk + chunk) * kHeadDim + 16 * dt + ln] = o;
    }
  }
  if (w == 0 && ln == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kb + i;
      if (g < G) {
        part_ml[(((size_t)(qrow0 + g)) * nchunk + chunk) * 2] = m[i];
        part_ml[(((size_t)(qrow0 + g)) * nchunk + chunk) * 2 + 1] = l[i];
      }
    }
}

// one workgroup of 128 threads per query row: o[n] = sum_c e^(m_c - m) o_c[n]
// / sum_c e^(m_c - m) l_c, chunks in order
__global__ __launch_bounds__(kHeadDim) void attn_combine_kernel(const float* __restrict__ part_o,
                                                                const float* __restrict__ part_ml, int nchunk,
                                                                uint16_t* __restrict__ out) {
  const size_t row = blockIdx.x;
  const int n = threadIdx.x;
  const float* ml = part_ml + row * nchunk * 2;
  float m = -INFINITY;
  for (int c = 0; c < nchunk; ++c) m = fmaxf(m, ml[2 * c]);
  float num = 0.f, den = 0.f;
  for (int c = 0; c < nchunk; ++c) {
    const float f = expf(ml[2 * c] - m);
    den = fmaf(f, ml[2 * c + 1], den);
    num = fmaf(f, part_o[(row * nchunk + c) * kHeadDim + n], num);
  }
  out[row * kHeadDim + n] = float_to_half_bits(num / den);
}

}  // namespace

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
  hipLaunchKernelGGL(attn_msd_chunk_kernel, dim3(nchunk, Hkv, B), dim3(kAttnThreads), 0, s, qsl, qsc, MQ, Hq, Hkv, L,
                     kp, ks, kz, vtp, vs, vz, po, pm);
  st = check_launch("attn_msd_chunk");
  if (st != 0) return st;
  hipLaunchKernelGGL(attn_combine_kernel, dim3(MQ), dim3(kHeadDim), 0, s, po, pm, nchunk, out);
  return check_launch("attn_combine");
}

}  // namespace w4

// Decode-shaped W4 product y[M][N] = x[M][K] . W' for 1 <= M <= 32.
//
// The weight stream dominates: every packed byte is read once from HBM with
// wide loads and turned into matrix-core operands in registers.  Dequantization
// is "after per-group mpGEMM" ("MixPE: Quantization and Hardware Co-design for
// Efficient LLM Inference", Abstract): each group's partial product is formed
// from the raw codes and multiplied by the group scale once.  NF4 levels come
// from a small table in LDS, as the "Fast NF4 Dequantization Kernels for Large
// Language Model Inference" page (Abstract) keeps its codebook in shared
// memory; here the table is indexed by a whole byte, so one lookup yields the
// pair of fp16 levels of two adjacent weights.
//
// Work split.  A workgroup owns 16*RT weight rows; its NW waves take the K
// groups round-robin (wave w: groups w, w+NW, ...), so together they sweep each
// row contiguously.  Partial sums meet in LDS at the end.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_f16).  The weight rows are the MFMA
// "n" dimension, tokens the "m" dimension.  Lane l serves row n = l%16 and
// k-block kb = l/16; per group it loads LB contiguous packed bytes (2*LB
// codes) starting at k = g*G + kb*2*LB, with G = 8*LB, so each group is one
// load per lane and the group boundary never splits an MFMA.
//
// INT4 operands.  A code q in the low nibble of an fp16 lane is the subnormal
// value q * 2^-24 exactly, and in bits 4..7 it is q * 2^-20; masking the packed
// word therefore yields exact fp16 operands in 5 VALU ops per 8 codes, with no
// offset to cancel.  The odd-position codes (2^-20) meet activations pre-scaled
// by 1/16, so every product is x*q*2^-24.  The zero point is applied with the
// group's activation sum: y += s * (2^24 * sum x*q - z * sum x), where sum x
// comes from the same activation operands times a constant B.
#include "w4_device.h"
#include "w4_internal.h"

#include <cstdlib>

namespace w4 {
namespace {

constexpr int kGemvMaxThreads = 512;

// fp16 pair constants
constexpr uint32_t kHalfOnePair = 0x3C003C00u;      // (1.0, 1.0)
constexpr uint32_t kHalfSixteenPair = 0x4C004C00u;  // (16.0, 16.0)
constexpr uint32_t kHalfSixteenthPair = 0x2C002C00u;  // (1/16, 1/16)

__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, b));
}

// Interleave the low (sel 0x05040100) or high (0x07060302) fp16 halves of two
// activation words: result = half(a) | half(b) << 16.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

template <int LB>
struct XWords {
  static constexpr int kU32 = LB;  // 2*LB halves = LB words
  uint32_t w[kU32];
};

template <int LB>
__device__ __forceinline__ void load_x(XWords<LB>& xw, const uint16_t* __restrict__ x, int M, int K,
                                       int m, int k0) {
  if (m < M) {
    const u32x4* p = reinterpret_cast<const u32x4*>(x + (size_t)m * K + k0);
#pragma unroll
    for (int v = 0; v < LB / 4; ++v) {
      const u32x4 t = p[v];
      xw.w[4 * v + 0] = t.x;
      xw.w[4 * v + 1] = t.y;
      xw.w[4 * v + 2] = t.z;
      xw.w[4 * v + 3] = t.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < LB; ++i) xw.w[i] = 0u;
  }
}

template <int LB>
struct WWords {
  uint32_t w[LB / 4];
};

template <int LB>
__device__ __forceinline__ void load_w(WWords<LB>& ww, const uint8_t* __restrict__ p) {
  if constexpr (LB == 16) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    ww.w[0] = t.x;
    ww.w[1] = t.y;
    ww.w[2] = t.z;
    ww.w[3] = t.w;
  } else {
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    ww.w[0] = t.x;
    ww.w[1] = t.y;
  }
}

template <int FMT, int LB, int MT, int RT>
__global__ __launch_bounds__(kGemvMaxThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero,
    uint16_t* __restrict__ y) {
  constexpr int G = 8 * LB;
  constexpr int NU = LB / 4;   // packed words per lane per group
  constexpr int NP = NU / 2;   // INT4: (even, odd) MFMA pairs per group
  extern __shared__ float red[];  // [NW][RT][MT][4][64]
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];

  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int nw = blockDim.x / kWave;
  const int ln = lane % 16;  // weight row within a row tile; token row for A
  const int kb = lane / 16;
  const int ng = K / G;
  const int row0 = blockIdx.x * (16 * RT);

  if constexpr (FMT == 1) {
    for (int b = threadIdx.x; b < 256; b += blockDim.x)
      lut[b] = (uint32_t)float_to_half_bits(nf4_level(b & 15)) |
               ((uint32_t)float_to_half_bits(nf4_level(b >> 4)) << 16);
    __syncthreads();
  }

  f32x4 C[RT][MT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < MT; ++t) C[rt][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  bool row_ok[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) row_ok[rt] = (row0 + rt * 16) < N;

  const size_t row_bytes = (size_t)K / 2;

  for (int g = wave; g < ng; g += nw) {
    const int k0 = g * G + kb * 2 * LB;
    // ---- activation operands for this group
    XWords<LB> xw[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) load_x<LB>(xw[t], x, M, K, t * 16 + ln, k0);
    WWords<LB> ww[RT];
    uint16_t sc[RT], zc[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int n = row0 + rt * 16 + ln;
      if (row_ok[rt]) {
        load_w<LB>(ww[rt], packed + (size_t)n * row_bytes + (size_t)g * (G / 2) + kb * LB);
        sc[rt] = scale[(size_t)n * ng + g];
        if constexpr (FMT == 0) zc[rt] = zero[(size_t)n * ng + g];
      } else {
#pragma unroll
        for (int u = 0; u < NU; ++u) ww[rt].w[u] = 0u;
        sc[rt] = 0;
        zc[rt] = 0;
      }
    }

    if constexpr (FMT == 0) {
      // A operands: even-position activations as loaded, odd ones scaled by 1/16.
      u32x4 AE[MT][NP], AO[MT][NP];
      f32x4 sx[MT];
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        sx[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const uint32_t* X = xw[t].w + 8 * p;
          AE[t][p] = u32x4{pair_lo(X[0], X[2]), pair_lo(X[1], X[3]), pair_lo(X[4], X[6]),
                           pair_lo(X[5], X[7])};
          AO[t][p] = u32x4{pk_mul_f16(pair_hi(X[0], X[2]), kHalfSixteenthPair),
                           pk_mul_f16(pair_hi(X[1], X[3]), kHalfSixteenthPair),
                           pk_mul_f16(pair_hi(X[4], X[6]), kHalfSixteenthPair),
                           pk_mul_f16(pair_hi(X[5], X[7]), kHalfSixteenthPair)};
          sx[t] = mfma_f16(AE[t][p], u32x4{kHalfOnePair, kHalfOnePair, kHalfOnePair, kHalfOnePair}, sx[t]);
          sx[t] = mfma_f16(AO[t][p], u32x4{kHalfSixteenPair, kHalfSixteenPair, kHalfSixteenPair,
                                           kHalfSixteenPair}, sx[t]);
        }
      }
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        u32x4 BE[NP], BO[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const uint32_t v0 = ww[rt].w[2 * p], v1 = ww[rt].w[2 * p + 1];
          const uint32_t v0s = v0 >> 8, v1s = v1 >> 8;
          BE[p] = u32x4{v0 & 0x000F000Fu, v0s & 0x000F000Fu, v1 & 0x000F000Fu, v1s & 0x000F000Fu};
          BO[p] = u32x4{v0 & 0x00F000F0u, v0s & 0x00F000F0u, v1 & 0x00F000F0u, v1s & 0x00F000F0u};
        }
        const float s = half_bits_to_float(sc[rt]);
        const float s24 = s * 16777216.0f;
        const float nsz = -s * half_bits_to_float(zc[rt]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            acc = mfma_f16(AE[t][p], BE[p], acc);
            acc = mfma_f16(AO[t][p], BO[p], acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) C[rt][t][i] = fmaf(s24, acc[i], fmaf(nsz, sx[t][i], C[rt][t][i]));
        }
      }
    } else {
      // NF4: natural k order on both operands; byte-indexed level-pair table.
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) {
        u32x4 B[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const uint32_t v = ww[rt].w[u];
          B[u] = u32x4{lut[v & 0xFFu], lut[(v >> 8) & 0xFFu], lut[(v >> 16) & 0xFFu], lut[v >> 24]};
        }
        const float a = half_bits_to_float(sc[rt]);
#pragma unroll
        for (int t = 0; t < MT; ++t) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int u = 0; u < NU; ++u) {
            const uint32_t* X = xw[t].w + 4 * u;
            acc = mfma_f16(u32x4{X[0], X[1], X[2], X[3]}, B[u], acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) C[rt][t][i] = fmaf(a, acc[i], C[rt][t][i]);
        }
      }
    }
  }

  // ---- cross-wave reduction through LDS, then fp16 store
  constexpr int kTile = RT * MT * 256;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave * kTile + ((rt * MT + t) * 4 + i) * 64 + lane] = C[rt][t][i];
  __syncthreads();
  for (int e = threadIdx.x; e < kTile; e += blockDim.x) {
    float sum = 0.f;
    for (int w = 0; w < nw; ++w) sum += red[w * kTile + e];
    const int l = e % 64;
    const int i = (e / 64) % 4;
    const int t = (e / 256) % MT;
    const int rt = e / (256 * MT);
    const int n = row0 + rt * 16 + l % 16;
    const int m = t * 16 + 4 * (l / 16) + i;
    if (m < M && n < N) y[(size_t)m * N + n] = float_to_half_bits(sum);
  }
}

struct GemvConfig {
  int rt;
  int nw;
};

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

GemvConfig choose_gemv(int M, int K, int N, int G) {
  GemvConfig c;
  const int tiles = N / 16;
  c.rt = tiles >= 2048 ? 2 : 1;
  const int ng = K / G;
  c.nw = ng >= 8 ? 8 : (ng >= 4 ? 4 : (ng >= 2 ? 2 : 1));
  (void)M;
  const int rt = env_int("W4_GEMV_RT", 0);
  const int nw = env_int("W4_GEMV_NW", 0);
  if (rt == 1 || rt == 2 || rt == 4) c.rt = rt;
  if (nw >= 1 && nw <= kGemvMaxThreads / kWave) c.nw = nw;
  return c;
}

template <int FMT, int LB, int MT>
int launch_rt(const GemvConfig& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
              const uint16_t* scale, const uint16_t* zero, uint16_t* y, hipStream_t s) {
  const dim3 block(c.nw * kWave);
  const dim3 grid((unsigned)((N + 16 * c.rt - 1) / (16 * c.rt)));
  const size_t lds = (size_t)c.nw * c.rt * MT * 256 * sizeof(float);
  switch (c.rt) {
    case 1:
      hipLaunchKernelGGL((gemv_kernel<FMT, LB, MT, 1>), grid, block, lds, s, x, M, K, N, packed, scale, zero, y);
      break;
    case 2:
      hipLaunchKernelGGL((gemv_kernel<FMT, LB, MT, 2>), grid, block, lds, s, x, M, K, N, packed, scale, zero, y);
      break;
    default:
      hipLaunchKernelGGL((gemv_kernel<FMT, LB, MT, 4>), grid, block, lds, s, x, M, K, N, packed, scale, zero, y);
      break;
  }
  return check_launch("gemv");
}

template <int FMT, int LB>
int launch_mt(const GemvConfig& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
              const uint16_t* scale, const uint16_t* zero, uint16_t* y, hipStream_t s) {
  if (M <= 16) return launch_rt<FMT, LB, 1>(c, x, M, K, N, packed, scale, zero, y, s);
  return launch_rt<FMT, LB, 2>(c, x, M, K, N, packed, scale, zero, y, s);
}

}  // namespace

int launch_gemv(const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                const uint16_t* scale, const uint16_t* zero, int G, int fmt, uint16_t* y,
                hipStream_t s) {
  const GemvConfig c = choose_gemv(M, K, N, G);
  if (fmt == 0) {
    if (G == 64) return launch_mt<0, 8>(c, x, M, K, N, packed, scale, zero, y, s);
    return launch_mt<0, 16>(c, x, M, K, N, packed, scale, zero, y, s);
  }
  if (G == 64) return launch_mt<1, 8>(c, x, M, K, N, packed, scale, zero, y, s);
  return launch_mt<1, 16>(c, x, M, K, N, packed, scale, zero, y, s);
}

}  // namespace w4

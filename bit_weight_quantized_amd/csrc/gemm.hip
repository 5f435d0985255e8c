// Prefill-shaped W4 products on the matrix cores, three ways (the three
// paths the pages compare):
//
//  PATH_DQ  dequantize-then-multiply: each weight becomes fp16 s*(q-z) (INT4)
//           or c[idx]*a (NF4) in registers, then fp16 MFMA accumulates
//           straight into the output tile -- the "dequantization baseline" of
//           the "Multi-Scale Dequant ..." and "Fast NF4 Dequantization ..."
//           pages (Abstracts).
//  PATH_PS  post-scaled: the integer codes (q-z), or the NF4 levels c[idx],
//           enter fp16 MFMA unscaled; each group's fp32 partial tile is
//           multiplied by the group scale once ("MixPE: Quantization and
//           Hardware Co-design for Efficient LLM Inference", Abstract:
//           dequantization after per-group mpGEMM).
//  PATH_MSD Multi-Scale Dequant: the activations arrive as int8 slices; the
//           4-bit codes are widened to int8 with mask/shift only (no
//           conversion to a floating type) and meet every slice on the int8
//           matrix cores, the same weight operand serving both slices; group
//           scales, zero points and token scales are applied after the
//           integer accumulation of each group.
//
// Tiling.  A workgroup of 4 waves (2 x 2) owns a BM x BN output tile, BM = 128
// rows of tokens, BN = 32 * NT columns; each wave owns 64 x 16*NT.  The K loop
// steps one quantization group at a time: the group's activation tile, packed
// weight tile, scales/zeros (and for MSD the slice sums) are staged in LDS,
// while the next group's tiles are already loading into registers.
//
// Operand order.  INT4 codes are unpacked in the order the cheapest mask/shift
// sequence produces them (for fp16: (k0,k4),(k1,k5),(k2,k6),(k3,k7) per 8
// codes; for int8: even codes then odd codes per 8), and the activation tile
// is permuted the same way once, when it is written to LDS.  A dot product is
// invariant under a common permutation of its terms.
//
// INT4 post-scaled operands are exact: the masked code q in the low bits of an
// fp16 lane is the subnormal q * 2^-24, and q - z is formed by one packed
// subtraction of subnormals (exact), so the group's fp32 partial is
// 2^-24 * sum x (q - z) and is scaled by s * 2^24.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {
namespace {

constexpr int kGemmThreads = 256;
constexpr int kBM = 128;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_sub_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) - __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

template <int PATH>
struct PathTraits;

// LDS tile geometry per path.  Row strides are padded by 16 bytes so the 16
// rows one fragment read touches fall in different banks.
template <int PATH, int LB, int NT, int NS>
struct GemmGeom {
  static constexpr int G = 8 * LB;
  static constexpr int BN = 32 * NT;
  static constexpr int A_ELEM = PATH == 2 ? 1 : 2;                  // bytes per activation element
  static constexpr int A_STRIDE = G * A_ELEM + 16;                  // bytes per tile row
  static constexpr int A_BYTES = NS * kBM * A_STRIDE;
  static constexpr int B_STRIDE = G / 2 + 16;
  static constexpr int B_BYTES = BN * B_STRIDE;
  static constexpr int OFF_B = A_BYTES;
  static constexpr int OFF_S = OFF_B + B_BYTES;                     // scale, zero bits per column
  static constexpr int OFF_T = OFF_S + BN * 4;                      // MSD: per-row fp32 T, int SA_j
  static constexpr int LDS = OFF_T + (PATH == 2 ? kBM * 4 * (1 + NS) : 0);
  static constexpr int A_CHUNKS = NS * kBM * G * A_ELEM / 16;       // 16-byte global chunks per group
  static constexpr int B_CHUNKS = BN * (G / 2) / 16;
  static constexpr int A_PER_T = A_CHUNKS / kGemmThreads;
  static constexpr int B_PER_T = (B_CHUNKS + kGemmThreads - 1) / kGemmThreads;
};

template <int PATH, int FMT, int LB, int NT, int NS>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const void* __restrict__ a_src, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    const float* __restrict__ tok_scale, const int32_t* __restrict__ gsum, int32_t* __restrict__ acc_out) {
  using Geo = GemmGeom<PATH, LB, NT, NS>;
  constexpr int G = Geo::G;
  constexpr int BN = Geo::BN;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave % 2, wn = wave / 2;
  const int ln = lane % 16, kb = lane / 16;
  const int n0 = blockIdx.x * BN;
  const int m0 = blockIdx.y * kBM;
  const int ng = K / G;
  const size_t row_bytes = (size_t)K / 2;

  if constexpr (FMT == 1) {
    for (int b = tid; b < 256; b += kGemmThreads)
      lut[b] = (uint32_t)float_to_half_bits(nf4_level(b & 15)) |
               ((uint32_t)float_to_half_bits(nf4_level(b >> 4)) << 16);
  }

  // ---- global -> register prefetch of one group's tiles
  u32x4 ra[Geo::A_PER_T];
  u32x4 rb[Geo::B_PER_T];
  uint16_t rs = 0, rz = 0;   // thread t < BN: column n0 + t
  int32_t rsa[NS];           // MSD, thread t < BM: slice sums of row m0 + t
  auto prefetch = [&](int g) {
#pragma unroll
    for (int i = 0; i < Geo::A_PER_T; ++i) {
      const int c = tid + i * kGemmThreads;
      if constexpr (PATH == 2) {
        constexpr int per_row = G / 16;
        const int j = c / (kBM * per_row);
        const int rem = c - j * kBM * per_row;
        const int r = rem / per_row, cc = rem - r * per_row;
        const int8_t* src = static_cast<const int8_t*>(a_src) + ((size_t)j * M + min(m0 + r, M - 1)) * K +
                            (size_t)g * G + cc * 16;
        ra[i] = *reinterpret_cast<const u32x4*>(src);
      } else {
        constexpr int per_row = G / 8;
        const int r = c / per_row, cc = c - r * per_row;
        const uint16_t* src =
            static_cast<const uint16_t*>(a_src) + (size_t)min(m0 + r, M - 1) * K + (size_t)g * G + cc * 8;
        ra[i] = *reinterpret_cast<const u32x4*>(src);
      }
    }
#pragma unroll
    for (int i = 0; i < Geo::B_PER_T; ++i) {
      constexpr int per_row = G / 32;
      const int c = min(tid + i * kGemmThreads, Geo::B_CHUNKS - 1);
      const int r = c / per_row, cc = c - r * per_row;
      rb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
          packed + (size_t)min(n0 + r, N - 1) * row_bytes + (size_t)g * (G / 2) + cc * 16));
    }
    {
      const size_t o = (size_t)min(n0 + min(tid, BN - 1), N - 1) * ng + g;
      rs = scale[o];
      if constexpr (FMT == 0) rz = zero[o];
    }
    if constexpr (PATH == 2) {
      const int r = min(m0 + min(tid, kBM - 1), M - 1);
#pragma unroll
      for (int j = 0; j < NS; ++j) rsa[j] = gsum[((size_t)j * M + r) * ng + g];
    }
  };

  // per-token ratio s2/s1 (MSD): for the 16 rows this lane's accumulators hold
  float rr[4][4];
  if constexpr (PATH == 2) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = min(m0 + wm * 64 + mt * 16 + 4 * kb + i, M - 1);
        const float s1 = tok_scale[m];
        rr[mt][i] = (NS == 2 && s1 != 0.f) ? tok_scale[(size_t)M + m] / s1 : 0.f;
      }
  }

  // ---- registers -> LDS (activation permutation applied here)
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < Geo::A_PER_T; ++i) {
      const int c = tid + i * kGemmThreads;
      u32x4 v = ra[i];
      unsigned char* dst;
      if constexpr (PATH == 2) {
        constexpr int per_row = G / 16;
        const int j = c / (kBM * per_row);
        const int rem = c - j * kBM * per_row;
        const int r = rem / per_row, cc = rem - r * per_row;
        dst = smem + (j * kBM + r) * Geo::A_STRIDE + cc * 16;
        // bytes (0,2,4,6 | 1,3,5,7) of each 8: even codes, then odd codes
        v = u32x4{perm_b32(v.y, v.x, 0x06040200u), perm_b32(v.y, v.x, 0x07050301u),
                  perm_b32(v.w, v.z, 0x06040200u), perm_b32(v.w, v.z, 0x07050301u)};
      } else {
        constexpr int per_row = G / 8;
        const int r = c / per_row, cc = c - r * per_row;
        dst = smem + r * Geo::A_STRIDE + cc * 16;
        if constexpr (FMT == 0)  // (x0,x4),(x1,x5),(x2,x6),(x3,x7)
          v = u32x4{pair_lo(v.x, v.z), pair_hi(v.x, v.z), pair_lo(v.y, v.w), pair_hi(v.y, v.w)};
      }
      *reinterpret_cast<u32x4*>(dst) = v;
    }
#pragma unroll
    for (int i = 0; i < Geo::B_PER_T; ++i) {
      constexpr int per_row = G / 32;
      const int c = tid + i * kGemmThreads;
      if (c < Geo::B_CHUNKS) {
        const int r = c / per_row, cc = c - r * per_row;
        *reinterpret_cast<u32x4*>(smem + Geo::OFF_B + r * Geo::B_STRIDE + cc * 16) = rb[i];
      }
    }
    if (tid < BN) {
      reinterpret_cast<uint16_t*>(smem + Geo::OFF_S)[tid] = rs;
      reinterpret_cast<uint16_t*>(smem + Geo::OFF_S)[BN + tid] = rz;
    }
    if constexpr (PATH == 2) {
      if (tid < kBM) {
        const int m = min(m0 + tid, M - 1);
        const float s1 = tok_scale[m];
        const float r = (NS == 2 && s1 != 0.f) ? tok_scale[(size_t)M + m] / s1 : 0.f;
        float t = (float)rsa[0];
        if constexpr (NS == 2) t = fmaf(r, (float)rsa[1], t);
        reinterpret_cast<float*>(smem + Geo::OFF_T)[tid] = t;
#pragma unroll
        for (int j = 0; j < NS; ++j) reinterpret_cast<int32_t*>(smem + Geo::OFF_T)[kBM * (1 + j) + tid] = rsa[j];
      }
    }
  };

  f32x4 C[4][NT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) C[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  prefetch(0);
  for (int g = 0; g < ng; ++g) {
    __syncthreads();  // previous group's compute is done with LDS
    stash();
    __syncthreads();
    prefetch(min(g + 1, ng - 1));  // unconditional: the last group is fetched twice

    const uint16_t* s_lds = reinterpret_cast<const uint16_t*>(smem + Geo::OFF_S);
    if constexpr (PATH != 2) {
      f32x4 acc[4][NT];
      if constexpr (PATH == 1) {
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // per-column (lane) constants of this group
      uint32_t zz[NT], sp[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = wn * 16 * NT + nt * 16 + ln;
        const uint32_t sb = s_lds[col];
        sp[nt] = sb | (sb << 16);  // (s, s) fp16 pair
        if constexpr (FMT == 0) {
          const uint32_t z = (uint32_t)half_bits_to_float(s_lds[BN + col]);  // integer 0..15
          // PS: (z, z) * 2^-24 as subnormal fp16; DQ: (1024 + z, 1024 + z)
          zz[nt] = PATH == 1 ? (z | (z << 16)) : ((0x6400u | z) | ((0x6400u | z) << 16));
        }
      }
#pragma unroll
      for (int ks = 0; ks < G / 32; ++ks) {
        u32x4 A[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          A[mt] = *reinterpret_cast<const u32x4*>(smem + (wm * 64 + mt * 16 + ln) * Geo::A_STRIDE +
                                                  (ks * 32 + 8 * kb) * 2);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = wn * 16 * NT + nt * 16 + ln;
          const uint32_t v =
              *reinterpret_cast<const uint32_t*>(smem + Geo::OFF_B + col * Geo::B_STRIDE + ks * 16 + 4 * kb);
          u32x4 B;
          if constexpr (FMT == 0) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const uint32_t q = (v >> (4 * j)) & 0x000F000Fu;
              if constexpr (PATH == 1) {
                w[j] = pk_sub_f16(q, zz[nt]);  // (q - z) * 2^-24, exact
              } else {
                w[j] = pk_mul_f16(pk_sub_f16(q | 0x64006400u, zz[nt]), sp[nt]);  // fp16(s * (q - z))
              }
            }
            B = u32x4{w[0], w[1], w[2], w[3]};
          } else {
            B = u32x4{lut[v & 0xFFu], lut[(v >> 8) & 0xFFu], lut[(v >> 16) & 0xFFu], lut[v >> 24]};
            if constexpr (PATH == 0) B = u32x4{pk_mul_f16(B.x, sp[nt]), pk_mul_f16(B.y, sp[nt]),
                                               pk_mul_f16(B.z, sp[nt]), pk_mul_f16(B.w, sp[nt])};
          }
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            if constexpr (PATH == 1) acc[mt][nt] = mfma_f16(A[mt], B, acc[mt][nt]);
            else C[mt][nt] = mfma_f16(A[mt], B, C[mt][nt]);
          }
        }
      }
      if constexpr (PATH == 1) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = wn * 16 * NT + nt * 16 + ln;
          float sf = half_bits_to_float(s_lds[col]);
          if constexpr (FMT == 0) sf *= 16777216.0f;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) C[mt][nt][i] = fmaf(sf, acc[mt][nt][i], C[mt][nt][i]);
        }
      }
    } else {
      // ---- MSD: int8 slices x int8 codes, int32 per group
      i32x4 D[NS][4][NT];
#pragma unroll
      for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) D[j][mt][nt] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int ks = 0; ks < G / 64; ++ks) {
        u32x4 A[NS][4];
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            A[j][mt] = *reinterpret_cast<const u32x4*>(smem + (j * kBM + wm * 64 + mt * 16 + ln) * Geo::A_STRIDE +
                                                       ks * 64 + 16 * kb);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = wn * 16 * NT + nt * 16 + ln;
          const u32x2 v =
              *reinterpret_cast<const u32x2*>(smem + Geo::OFF_B + col * Geo::B_STRIDE + ks * 32 + 8 * kb);
          const u32x4 B{v.x & 0x0F0F0F0Fu, (v.x >> 4) & 0x0F0F0F0Fu, v.y & 0x0F0F0F0Fu, (v.y >> 4) & 0x0F0F0F0Fu};
#pragma unroll
          for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) D[j][mt][nt] = mfma_i8(A[j][mt], B, D[j][mt][nt]);
        }
      }
      // group epilogue: C' += s * (D1 + r * D2) - s * z * (SA1 + r * SA2)
      const float* t_lds = reinterpret_cast<const float*>(smem + Geo::OFF_T);
      const int32_t* sa_lds = reinterpret_cast<const int32_t*>(smem + Geo::OFF_T);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = wn * 16 * NT + nt * 16 + ln;
        const float sv = half_bits_to_float(s_lds[col]);
        const float zv = half_bits_to_float(s_lds[BN + col]);
        const float nsz = -sv * zv;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const int rloc = wm * 64 + mt * 16 + 4 * kb;
          const f32x4 T = *reinterpret_cast<const f32x4*>(t_lds + rloc);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float e = (float)D[0][mt][nt][i];
            if constexpr (NS == 2) e = fmaf(rr[mt][i], (float)D[1][mt][nt][i], e);
            C[mt][nt][i] = fmaf(sv, e, fmaf(nsz, T[i], C[mt][nt][i]));
          }
          if (acc_out) {  // debug output: exact integer per-group products, zero point folded
            const int n = n0 + col;
            const int z = (int)zv;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = m0 + rloc + i;
              if (m < M && n < N) {
#pragma unroll
                for (int j = 0; j < NS; ++j)
                  acc_out[(((size_t)j * M + m) * ng + g) * N + n] =
                      D[j][mt][nt][i] - z * sa_lds[kBM * (1 + j) + rloc + i];
              }
            }
          }
        }
      }
    }
  }

  // ---- store: y = C (MSD: times the token's first-slice scale)
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 64 + mt * 16 + 4 * kb + i;
      if (m >= M) continue;
      float rs1 = 1.f;
      if constexpr (PATH == 2) rs1 = tok_scale[m];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + wn * 16 * NT + nt * 16 + ln;
        if (n < N) y[(size_t)m * N + n] = float_to_half_bits(C[mt][nt][i] * rs1);
      }
    }
}

template <int PATH, int FMT, int LB, int NT, int NS>
int launch_one(const void* a, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
               const uint16_t* zero, uint16_t* y, const float* tok_scale, const int32_t* gsum, int32_t* acc_out,
               hipStream_t s) {
  using Geo = GemmGeom<PATH, LB, NT, NS>;
  static_assert(Geo::A_CHUNKS % kGemmThreads == 0, "activation tile must split evenly over the threads");
  const dim3 grid((unsigned)((N + Geo::BN - 1) / Geo::BN), (unsigned)((M + kBM - 1) / kBM));
  hipLaunchKernelGGL((gemm_kernel<PATH, FMT, LB, NT, NS>), grid, dim3(kGemmThreads), Geo::LDS, s, a, M, K, N, packed,
                     scale, zero, y, tok_scale, gsum, acc_out);
  return check_launch(PATH == 2 ? "gemm_msd" : "gemm");
}

}  // namespace

int launch_gemm(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                const uint16_t* zero, int G, int fmt, int mode, uint16_t* y, hipStream_t s) {
  constexpr int NT = 4;
#define W4_GEMM_CASE(PATH, FMT, LB)                                                                          \
  return launch_one<PATH, FMT, LB, NT, 1>(x, M, K, N, packed, scale, zero, y, nullptr, nullptr, nullptr, s)
  if (mode == 0) {
    if (fmt == 0) {
      if (G == 64) W4_GEMM_CASE(0, 0, 8);
      W4_GEMM_CASE(0, 0, 16);
    }
    if (G == 64) W4_GEMM_CASE(0, 1, 8);
    W4_GEMM_CASE(0, 1, 16);
  }
  if (fmt == 0) {
    if (G == 64) W4_GEMM_CASE(1, 0, 8);
    W4_GEMM_CASE(1, 0, 16);
  }
  if (G == 64) W4_GEMM_CASE(1, 1, 8);
  W4_GEMM_CASE(1, 1, 16);
#undef W4_GEMM_CASE
}

size_t decomp_workspace_bytes(int M, int K, int G, int nslices) {
  const size_t slices = ((size_t)nslices * M * K + 255) / 256 * 256;
  const size_t scales = ((size_t)nslices * M * sizeof(float) + 255) / 256 * 256;
  const size_t sums = (size_t)nslices * M * (K / G) * sizeof(int32_t);
  return slices + scales + sums;
}

int launch_gemm_decomp(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                       const uint16_t* zero, int G, int nslices, uint16_t* y, int8_t* slices, float* tok_scale,
                       int32_t* gsum, int32_t* acc_out, hipStream_t s) {
  int st = launch_decompose(x, M, K, G, nslices, slices, tok_scale, gsum, s);
  if (st != 0) return st;
  constexpr int NT = 2;
  if (nslices == 1) {
    if (G == 64) return launch_one<2, 0, 8, NT, 1>(slices, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out, s);
    return launch_one<2, 0, 16, NT, 1>(slices, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out, s);
  }
  if (G == 64) return launch_one<2, 0, 8, NT, 2>(slices, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out, s);
  return launch_one<2, 0, 16, NT, 2>(slices, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out, s);
}

}  // namespace w4

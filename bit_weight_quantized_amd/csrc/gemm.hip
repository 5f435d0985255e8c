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
// steps one weight-tile column (128 K positions: one or two quantization
// groups) at a time: the step's activation tile, weight tiles, scales/zeros
// (and for MSD the slice sums) are stored to LDS while the next step's tiles
// are already loading into registers.
//
// Weight tiles.  The packed weights are stored as 1 KB tiles of 16 rows x 128
// K positions in which lane l finds its B operands in bytes 16 l .. 16 l + 15
// (word t: 8 codes of row l % 16 at K positions 32 t + 8 (l / 16) + 0..7).  A
// tile is copied to LDS as is and read back with one 16-byte load per lane.
//
// Operand order.  With the stored nibble order (even K positions in nibbles
// 0-3, odd in 4-7) the fp16 masks (w >> 4i) & 0x000F000F give the pairs
// (c0,c1),(c2,c3),... in K order, so INT4 activations are staged as they are.
// The int8 masks (bytes c0 c4 c1 c5 | c2 c6 c3 c7) and the NF4 byte table
// ((c0,c2),(c4,c6),(c1,c3),(c5,c7)) need the activation tile permuted the
// same way once, when it is written to LDS; a dot product is invariant under a
// common permutation of its terms.
//
// INT4 post-scaled operands are exact: the masked code q in the low bits of an
// fp16 lane is the subnormal q * 2^-24, and q - z is formed by one packed
// subtraction of subnormals (exact), so the group's fp32 partial is
// 2^-24 * sum x (q - z) and is scaled by s * 2^24.
//
// Block order.  Workgroups are dealt to the 8 XCDs round-robin; the kernel
// renumbers them so each XCD gets a contiguous run of output tiles, N fastest,
// and the token rows it shares stay in that XCD's L2.
#include "w4_device.h"
#include "w4_internal.h"

namespace w4 {
namespace {

constexpr int kGemmThreads = 256;
constexpr int kBM = 128;
constexpr int kStepK = 128;  // one weight-tile column per K step
constexpr int kXcds = 8;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_sub_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) - __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// LDS geometry per path.  Activation planes are padded by one 16-byte row so
// the staging writes (16 planes per token row) fall in different banks.
template <int PATH, int NT, int NS, int GPT>
struct GemmGeom {
  static constexpr int BN = 32 * NT;
  static constexpr int A_PLANES = PATH == 2 ? 8 : 16;  // fp16: chunk c of 8; int8: (product u, k-block j)
  static constexpr int A_PLANE = (kBM + 1) * 16;
  static constexpr int A_BYTES = (PATH == 2 ? NS : 1) * A_PLANES * A_PLANE;
  static constexpr int B_BYTES = (BN / 16) * 1024;
  static constexpr int OFF_B = A_BYTES;
  static constexpr int OFF_S = OFF_B + B_BYTES;          // [GPT][scale, zero][BN] fp16 bits
  static constexpr int OFF_T = OFF_S + GPT * 2 * BN * 2;  // MSD: T [GPT][BM] fp32, SA [GPT][NS][BM] int32
  static constexpr int OFF_R = OFF_T + (PATH == 2 ? GPT * kBM * 4 * (1 + NS) : 0);  // MSD: s2/s1 per row
  static constexpr int LDS = OFF_R + (PATH == 2 ? kBM * 4 : 0);
  static constexpr int A_UNITS = PATH == 2 ? NS * kBM * 8 : kBM * 16;  // 16-byte global chunks per step
  static constexpr int B_UNITS = (BN / 16) * 64;
  static constexpr int A_PER_T = A_UNITS / kGemmThreads;
  static constexpr int B_PER_T = (B_UNITS + kGemmThreads - 1) / kGemmThreads;
};

template <int PATH, int FMT, int GPT, int NT, int NS, bool DBG>
__global__ __launch_bounds__(kGemmThreads) void gemm_kernel(
    const void* __restrict__ a_src, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    const float* __restrict__ tok_scale, const int32_t* __restrict__ gsum, int32_t* __restrict__ acc_out) {
  using Geo = GemmGeom<PATH, NT, NS, GPT>;
  constexpr int BN = Geo::BN;
  constexpr int G = kStepK / GPT;
  constexpr int WPG = 4 / GPT;  // fp16 products (tile words) per group
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave % 2, wn = wave / 2;
  const int ln = lane % 16, kb = lane / 16;

  // XCD-aware renumbering (a bijection of [0, tiles))
  const int tiles_n = (N + BN - 1) / BN;
  const int tiles = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b % kXcds, idx = b / kXcds;
  const int per = tiles / kXcds, rem = tiles % kXcds;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
  const int n0 = (logical % tiles_n) * BN;
  const int m0 = (logical / tiles_n) * kBM;

  const int ng = K / G;
  const int KT = K / kStepK;
  const int ntile_last = N / 16 - 1;

  if constexpr (FMT == 1) {
    for (int i = tid; i < 256; i += kGemmThreads)
      lut[i] = (uint32_t)float_to_half_bits(nf4_level(i & 15)) |
               ((uint32_t)float_to_half_bits(nf4_level(i >> 4)) << 16);
  }

  // ---- global -> register prefetch of one K step
  u32x4 ra[Geo::A_PER_T];
  u32x4 rb[Geo::B_PER_T];
  uint16_t rs = 0, rz = 0;  // thread t < GPT*BN: group t / BN, column n0 + t % BN
  int32_t rsa[NS];          // MSD, thread t < GPT*BM: slice sums of group t / BM, row m0 + t % BM
  auto prefetch = [&](int kt) {
#pragma unroll
    for (int i = 0; i < Geo::A_PER_T; ++i) {
      const int u = tid + i * kGemmThreads;
      if constexpr (PATH == 2) {
        const int js = u / (kBM * 8);
        const int rem8 = u - js * kBM * 8;
        const int m = rem8 / 8, c = rem8 % 8;
        const int8_t* src = static_cast<const int8_t*>(a_src) + ((size_t)js * M + min(m0 + m, M - 1)) * K +
                            (size_t)kt * kStepK + c * 16;
        ra[i] = *reinterpret_cast<const u32x4*>(src);
      } else {
        const int m = u / 16, c = u % 16;
        const uint16_t* src =
            static_cast<const uint16_t*>(a_src) + (size_t)min(m0 + m, M - 1) * K + (size_t)kt * kStepK + c * 8;
        ra[i] = *reinterpret_cast<const u32x4*>(src);
      }
    }
#pragma unroll
    for (int i = 0; i < Geo::B_PER_T; ++i) {
      const int u = min(tid + i * kGemmThreads, Geo::B_UNITS - 1);
      const int t = u / 64, slot = u % 64;
      const size_t tile = (size_t)min(n0 / 16 + t, ntile_last) * KT + kt;
      rb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(packed + tile * 1024 + slot * 16));
    }
    {
      const int t = min(tid, GPT * BN - 1);
      const size_t o = (size_t)min(n0 + t % BN, N - 1) * ng + (size_t)kt * GPT + t / BN;
      rs = scale[o];
      if constexpr (FMT == 0) rz = zero[o];
    }
    if constexpr (PATH == 2) {
      const int t = min(tid, GPT * kBM - 1);
      const int r = min(m0 + t % kBM, M - 1);
#pragma unroll
      for (int j = 0; j < NS; ++j) rsa[j] = gsum[((size_t)j * M + r) * ng + (size_t)kt * GPT + t / kBM];
    }
  };

  // per-token ratio s2/s1 (MSD), one per tile row, in LDS (read after the
  // first barrier of the K loop)
  if constexpr (PATH == 2) {
    if (tid < kBM) {
      const int m = min(m0 + tid, M - 1);
      const float s1 = tok_scale[m];
      reinterpret_cast<float*>(smem + Geo::OFF_R)[tid] =
          (NS == 2 && s1 != 0.f) ? tok_scale[(size_t)M + m] / s1 : 0.f;
    }
  }

  // ---- registers -> LDS (activation permutation applied here)
  auto stash = [&]() {
#pragma unroll
    for (int i = 0; i < Geo::A_PER_T; ++i) {
      const int u = tid + i * kGemmThreads;
      const u32x4 v = ra[i];
      if constexpr (PATH == 2) {
        const int js = u / (kBM * 8);
        const int rem8 = u - js * kBM * 8;
        const int m = rem8 / 8, c = rem8 % 8;
        // K positions 16c .. 16c+15 of the step: product pu = c / 4, half h of
        // its 32-blocks, k-blocks jj and jj + 1; bytes reordered to the int8
        // masks' order x0 x4 x1 x5 x2 x6 x3 x7
        const int pu = c / 4, h = (c % 4) / 2, jj = 2 * (c % 2);
        unsigned char* base = smem + js * Geo::A_PLANES * Geo::A_PLANE + m * 16 + 8 * h;
        *reinterpret_cast<u32x2*>(base + (pu * 4 + jj) * Geo::A_PLANE) =
            u32x2{perm_b32(v.y, v.x, 0x05010400u), perm_b32(v.y, v.x, 0x07030602u)};
        *reinterpret_cast<u32x2*>(base + (pu * 4 + jj + 1) * Geo::A_PLANE) =
            u32x2{perm_b32(v.w, v.z, 0x05010400u), perm_b32(v.w, v.z, 0x07030602u)};
      } else {
        const int m = u / 16, c = u % 16;
        u32x4 q = v;  // INT4: the masks yield (c0,c1),(c2,c3),... -- K order, stored as is
        if constexpr (FMT == 1)  // NF4 level pairs of bytes 0..3: (x0,x2),(x4,x6),(x1,x3),(x5,x7)
          q = u32x4{pair_lo(v.x, v.y), pair_lo(v.z, v.w), pair_hi(v.x, v.y), pair_hi(v.z, v.w)};
        *reinterpret_cast<u32x4*>(smem + c * Geo::A_PLANE + m * 16) = q;
      }
    }
#pragma unroll
    for (int i = 0; i < Geo::B_PER_T; ++i) {
      const int u = tid + i * kGemmThreads;
      if (u < Geo::B_UNITS) *reinterpret_cast<u32x4*>(smem + Geo::OFF_B + u * 16) = rb[i];
    }
    if (tid < GPT * BN) {
      const int gi = tid / BN, col = tid % BN;
      reinterpret_cast<uint16_t*>(smem + Geo::OFF_S)[(gi * 2) * BN + col] = rs;
      reinterpret_cast<uint16_t*>(smem + Geo::OFF_S)[(gi * 2 + 1) * BN + col] = rz;
    }
    if constexpr (PATH == 2) {
      if (tid < GPT * kBM) {
        const int gi = tid / kBM, row = tid % kBM;
        const int m = min(m0 + row, M - 1);
        const float s1 = tok_scale[m];
        const float r = (NS == 2 && s1 != 0.f) ? tok_scale[(size_t)M + m] / s1 : 0.f;
        float t = (float)rsa[0];
        if constexpr (NS == 2) t = fmaf(r, (float)rsa[1], t);
        reinterpret_cast<float*>(smem + Geo::OFF_T)[gi * kBM + row] = t;
#pragma unroll
        for (int j = 0; j < NS; ++j)
          reinterpret_cast<int32_t*>(smem + Geo::OFF_T)[GPT * kBM + (gi * NS + j) * kBM + row] = rsa[j];
      }
    }
  };

  f32x4 C[4][NT];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) C[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint16_t* s_lds = reinterpret_cast<const uint16_t*>(smem + Geo::OFF_S);
  prefetch(0);
  for (int kt = 0; kt < KT; ++kt) {
    __syncthreads();  // the previous step's products are done with LDS
    stash();
    __syncthreads();
    prefetch(min(kt + 1, KT - 1));  // unconditional: the last step is fetched twice

    // this lane's 16 bytes of each of the wave's weight tiles
    u32x4 Bq[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      Bq[nt] = *reinterpret_cast<const u32x4*>(smem + Geo::OFF_B + (wn * NT + nt) * 1024 + lane * 16);

    if constexpr (PATH != 2) {
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
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
          const uint32_t sb = s_lds[(gi * 2) * BN + col];
          sp[nt] = sb | (sb << 16);  // (s, s) fp16 pair
          if constexpr (FMT == 0) {
            const uint32_t z = (uint32_t)half_bits_to_float(s_lds[(gi * 2 + 1) * BN + col]);  // 0..15
            // PS: (z, z) * 2^-24 as subnormal fp16; DQ: (1024 + z, 1024 + z)
            zz[nt] = PATH == 1 ? (z | (z << 16)) : ((0x6400u | z) | ((0x6400u | z) << 16));
          }
        }
#pragma unroll
        for (int w = gi * WPG; w < (gi + 1) * WPG; ++w) {
          u32x4 A[4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
            A[mt] = *reinterpret_cast<const u32x4*>(smem + (4 * w + kb) * Geo::A_PLANE + (wm * 64 + mt * 16 + ln) * 16);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const uint32_t v = Bq[nt][w];
            u32x4 B;
            if constexpr (FMT == 0) {
              uint32_t d[4];
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const uint32_t q = (v >> (4 * j)) & 0x000F000Fu;
                if constexpr (PATH == 1) {
                  d[j] = pk_sub_f16(q, zz[nt]);  // (q - z) * 2^-24, exact
                } else {
                  d[j] = pk_mul_f16(pk_sub_f16(q | 0x64006400u, zz[nt]), sp[nt]);  // fp16(s * (q - z))
                }
              }
              B = u32x4{d[0], d[1], d[2], d[3]};
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
            float sf = half_bits_to_float(s_lds[(gi * 2) * BN + col]);
            if constexpr (FMT == 0) sf *= 16777216.0f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) C[mt][nt][i] = fmaf(sf, acc[mt][nt][i], C[mt][nt][i]);
          }
        }
      }
    } else {
      // ---- MSD: int8 slices x int8 codes, exact int32 per group
      const float* t_lds = reinterpret_cast<const float*>(smem + Geo::OFF_T);
      const int32_t* sa_lds = reinterpret_cast<const int32_t*>(smem + Geo::OFF_T) + GPT * kBM;
      constexpr int UPG = 2 / GPT;  // int8 products (64 K positions each) per group
#pragma unroll
      for (int gi = 0; gi < GPT; ++gi) {
        i32x4 D[NS][4][NT];
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) D[j][mt][nt] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int pu = gi * UPG; pu < (gi + 1) * UPG; ++pu) {
          u32x4 A[NS][4];
#pragma unroll
          for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
              A[j][mt] = *reinterpret_cast<const u32x4*>(smem + j * Geo::A_PLANES * Geo::A_PLANE +
                                                         (pu * 4 + kb) * Geo::A_PLANE +
                                                         (wm * 64 + mt * 16 + ln) * 16);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const uint32_t w0 = Bq[nt][2 * pu], w1 = Bq[nt][2 * pu + 1];
            const u32x4 B{w0 & 0x0F0F0F0Fu, (w0 >> 4) & 0x0F0F0F0Fu, w1 & 0x0F0F0F0Fu, (w1 >> 4) & 0x0F0F0F0Fu};
#pragma unroll
            for (int j = 0; j < NS; ++j)
#pragma unroll
              for (int mt = 0; mt < 4; ++mt) D[j][mt][nt] = mfma_i8(A[j][mt], B, D[j][mt][nt]);
          }
        }
        // group epilogue: C' += s * (D1 + r * D2) - s * z * (SA1 + r * SA2)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int col = wn * 16 * NT + nt * 16 + ln;
          const float sv = half_bits_to_float(s_lds[(gi * 2) * BN + col]);
          const float zv = half_bits_to_float(s_lds[(gi * 2 + 1) * BN + col]);
          const float nsz = -sv * zv;
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            const int rloc = wm * 64 + mt * 16 + 4 * kb;
            const f32x4 T = *reinterpret_cast<const f32x4*>(t_lds + gi * kBM + rloc);
            const f32x4 rr = *reinterpret_cast<const f32x4*>(smem + Geo::OFF_R + rloc * 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float e = (float)D[0][mt][nt][i];
              if constexpr (NS == 2) e = fmaf(rr[i], (float)D[1][mt][nt][i], e);
              C[mt][nt][i] = fmaf(sv, e, fmaf(nsz, T[i], C[mt][nt][i]));
            }
            if constexpr (DBG) {  // debug output: exact integer per-group products, zero point folded
              const int n = n0 + col;
              const int z = (int)zv;
              const int g = kt * GPT + gi;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int m = m0 + rloc + i;
                if (m < M && n < N) {
#pragma unroll
                  for (int j = 0; j < NS; ++j)
                    acc_out[(((size_t)j * M + m) * ng + g) * N + n] =
                        D[j][mt][nt][i] - z * sa_lds[(gi * NS + j) * kBM + rloc + i];
                }
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

// ---------------------------------------------------------------------------
// fp16 matrix-core paths (PATH_DQ, PATH_PS), large tile: a workgroup of 8
// waves (2 x 4, two per SIMD: one wave alone cannot keep the matrix core
// busy) owns 256 tokens x 128 weight rows; each wave owns 128 x 32 (8 x 2
// products of 16 x 16), so every unpacked weight operand feeds 128 token
// rows.  The K step is one weight-tile column.  Both operand tiles of a
// step are copied global -> LDS by the load unit itself (16 bytes per lane,
// lane l's bytes landing at the instruction's LDS base + 16 l), double
// buffered: step k+1 is in flight while step k is computed, and one barrier
// per step hands the buffers over.  The activation tile is row-major in LDS
// (256 bytes per token row), 16-byte chunk c of row m at position c ^ (m % 16),
// which keeps both the fill and the operand reads free of bank conflicts.
// One workgroup per CU (its two buffers take most of the LDS).
constexpr int kF16BM = 256;
constexpr int kF16BN = 128;
constexpr int kF16Threads = 512;  // 8 waves: 2 (M) x 4 (N), two per SIMD
constexpr int kF16A = kF16BM * 256;            // activation tile bytes per stage
constexpr int kF16B = (kF16BN / 16) * 1024;    // weight tiles
constexpr int kF16S = 2 * 2 * kF16BN * 2;      // [group in step][scale, zero][BN] fp16 bits
constexpr int kF16Stage = kF16A + kF16B + kF16S;

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a raw buffer (offset = voff + soff) to lds_base +
// 16 * lane (lds_base wave-uniform).  Lanes whose voff lies past the buffer
// write zeros.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                              unsigned char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds_base, 16, voff, soff, 0, 0);
}

template <int PATH, int FMT, int GPT>
__global__ __launch_bounds__(kF16Threads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_f16_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y) {
  constexpr int G = kStepK / GPT;
  constexpr int WPG = 4 / GPT;  // products (tile words) per group
  constexpr int MT = 8, NT = 2;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave % 2, wn = wave / 2;  // wn = 0..3
  const int ln = lane % 16, kb = lane / 16;

  // XCD-aware renumbering (a bijection of [0, tiles))
  const int tiles_n = (N + kF16BN - 1) / kF16BN;
  const int tiles = gridDim.x;
  const int b = blockIdx.x;
  const int xcd = b % kXcds, idx = b / kXcds;
  const int per = tiles / kXcds, rem = tiles % kXcds;
  const int logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + idx;
  const int n0 = (logical % tiles_n) * kF16BN;
  const int m0 = (logical / tiles_n) * kF16BM;

  const int ng = K / G;
  const int KT = K / kStepK;
  const int ntile_last = N / 16 - 1;

  if constexpr (FMT == 1) {
    for (int i = tid; i < 256; i += kF16Threads)
      lut[i] = (uint32_t)float_to_half_bits(nf4_level(i & 15)) |
               ((uint32_t)float_to_half_bits(nf4_level(i >> 4)) << 16);
  }

  // ---- per-lane copy offsets (fixed for the whole K loop; the step adds a
  // scalar offset).  This wave fills token rows [32 wave, 32 wave + 32), 4 rows
  // per instruction, and weight tile `wave`.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(packed, (uint32_t)((size_t)N * (K / 2)));
  // instruction i covers rows 32 wave + 4 i + lane / 16; its swizzle depends on
  // i % 4 only, so four bases plus a row stride give every offset
  uint32_t voff_a4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wave * 32 + 4 * i + lane / 16;
    const int c = (lane % 16) ^ (row & 15);
    voff_a4[i] = (uint32_t)(m0 + row) * (uint32_t)(K * 2) + (uint32_t)c * 16;  // rows past M read zeros
  }
  const uint32_t row16_bytes = (uint32_t)K * 32;  // 16 token rows
  const uint32_t voff_b = (uint32_t)min(n0 / 16 + wave, ntile_last) * (uint32_t)KT * 1024 + (uint32_t)lane * 16;
  auto issue_step = [&](int kt, unsigned char* st) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      copy16_to_lds(xr, voff_a4[i % 4] + (uint32_t)(i / 4) * row16_bytes, (uint32_t)kt * 256,
                    st + (wave * 32 + 4 * i) * 256);
    copy16_to_lds(wr, voff_b, (uint32_t)kt * 1024, st + kF16A + wave * 1024);
  };
  // scales / zeros of a step: thread t < GPT * BN holds group t / BN, column t % BN
  auto load_scales = [&](int kt, uint16_t& rs, uint16_t& rz) {
    const int t = min(tid, GPT * kF16BN - 1);
    const size_t o = (size_t)min(n0 + t % kF16BN, N - 1) * ng + (size_t)kt * GPT + t / kF16BN;
    rs = scale[o];
    rz = FMT == 0 ? zero[o] : (uint16_t)0;
  };
  auto store_scales = [&](unsigned char* st, uint16_t rs, uint16_t rz) {
    if (tid < GPT * kF16BN) {
      const int gi = tid / kF16BN, col = tid % kF16BN;
      reinterpret_cast<uint16_t*>(st + kF16A + kF16B)[(gi * 2) * kF16BN + col] = rs;
      reinterpret_cast<uint16_t*>(st + kF16A + kF16B)[(gi * 2 + 1) * kF16BN + col] = rz;
    }
  };
  // operand-read offsets within a stage: word w of token tile mt at
  // a_off[w] + mt * 4096 (swizzled chunk 4w + kb of row wm*128 + mt*16 + ln)
  uint32_t a_off[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) a_off[w] = (uint32_t)(wm * 128 + ln) * 256 + ((uint32_t)((4 * w + kb) ^ ln) << 4);

  f32x4 C[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) C[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  {
    uint16_t rs, rz;
    issue_step(0, smem);
    load_scales(0, rs, rz);
    store_scales(smem, rs, rz);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    unsigned char* cur = smem + (kt & 1) * kF16Stage;
    unsigned char* nxt = smem + ((kt + 1) & 1) * kF16Stage;
    const bool more = kt + 1 < KT;
    uint16_t rs = 0, rz = 0;
    if (more) {
      issue_step(kt + 1, nxt);
      load_scales(kt + 1, rs, rz);
    }

    const uint16_t* s_lds = reinterpret_cast<const uint16_t*>(cur + kF16A + kF16B);
    u32x4 Bq[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      Bq[nt] = *reinterpret_cast<const u32x4*>(cur + kF16A + (wn * NT + nt) * 1024 + lane * 16);

    // Word by word: the next word's weight operands are unpacked while this
    // word's 16 products run; the second wave on the SIMD covers the LDS
    // latency of the fragment reads.
    float sfv[GPT][NT];      // PS: per-column scale (x 2^24 for INT4)
    uint32_t zzv[GPT][NT];   // INT4: zero-point pair
    uint32_t spv[GPT][NT];   // DQ: (s, s) pair
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = wn * 32 + nt * 16 + ln;
        const uint32_t sb = s_lds[(gi * 2) * kF16BN + col];
        spv[gi][nt] = sb | (sb << 16);
        sfv[gi][nt] = half_bits_to_float((uint16_t)sb) * (FMT == 0 ? 16777216.0f : 1.0f);
        zzv[gi][nt] = 0;
        if constexpr (FMT == 0) {
          const uint32_t z = (uint32_t)half_bits_to_float(s_lds[(gi * 2 + 1) * kF16BN + col]);  // 0..15
          // PS: (z, z) * 2^-24 as subnormal fp16; DQ: (1024 + z, 1024 + z)
          zzv[gi][nt] = PATH == 1 ? (z | (z << 16)) : ((0x6400u | z) | ((0x6400u | z) << 16));
        }
      }
    auto unpack = [&](u32x4 (&Bu)[NT], int w) {
      const int gi = w / WPG;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t v = Bq[nt][w];
        if constexpr (FMT == 0) {
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t q = (v >> (4 * j)) & 0x000F000Fu;  // (c_2j, c_2j+1) * 2^-24
            d[j] = PATH == 1 ? pk_sub_f16(q, zzv[gi][nt]) : pk_mul_f16(pk_sub_f16(q | 0x64006400u, zzv[gi][nt]), spv[gi][nt]);
          }
          Bu[nt] = u32x4{d[0], d[1], d[2], d[3]};
        } else {
          // table index (c_2j | c_2j+1 << 4) for the K-ordered pairs: even positions
          // sit in nibbles 0-3 and odd ones in 4-7, so fold bytes 2,3 onto 0,1
          const uint32_t lo = v & 0x0F0F0F0Fu, hi = (v >> 4) & 0x0F0F0F0Fu;
          const uint32_t il = lo | (lo >> 12), ih = hi | (hi >> 12);  // bytes 0,1: pairs (0,1),(4,5) / (2,3),(6,7)
          u32x4 L{lut[il & 0xFFu], lut[ih & 0xFFu], lut[(il >> 8) & 0xFFu], lut[(ih >> 8) & 0xFFu]};
          if constexpr (PATH == 0)
            L = u32x4{pk_mul_f16(L.x, spv[gi][nt]), pk_mul_f16(L.y, spv[gi][nt]), pk_mul_f16(L.z, spv[gi][nt]),
                      pk_mul_f16(L.w, spv[gi][nt])};
          Bu[nt] = L;
        }
      }
    };
    auto load_a = [&](u32x4 (&A)[MT], int w) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) A[mt] = *reinterpret_cast<const u32x4*>(cur + a_off[w] + mt * 4096);
    };

    f32x4 acc[MT][NT];  // PS: the group's partial products
    u32x4 B0[NT], B1[NT];
    unpack(B0, 0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x4(&Bc)[NT] = (w % 2 == 0) ? B0 : B1;
      u32x4(&Bn)[NT] = (w % 2 == 0) ? B1 : B0;
      u32x4 A[MT];
      load_a(A, w);
      if (w + 1 < 4) unpack(Bn, w + 1);  // next word's operands while this word's products run
      const bool first = (w % WPG) == 0;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          if constexpr (PATH == 1) acc[mt][nt] = mfma_f16(A[mt], Bc[nt], first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mt][nt]);
          else C[mt][nt] = mfma_f16(A[mt], Bc[nt], C[mt][nt]);
        }
      if constexpr (PATH == 1) {
        if ((w % WPG) == WPG - 1) {  // group complete: scale once
          const int gi = w / WPG;
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
#pragma unroll
              for (int i = 0; i < 4; ++i) C[mt][nt][i] = fmaf(sfv[gi][nt], acc[mt][nt][i], C[mt][nt][i]);
        }
      }
    }

    if (more) store_scales(nxt, rs, rz);
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies for the next step have landed
    __syncthreads();                // everyone's have, and nobody still reads this step's buffer
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 128 + mt * 16 + 4 * kb + i;
      if (m >= M) continue;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + wn * 32 + nt * 16 + ln;
        if (n < N) y[(size_t)m * N + n] = float_to_half_bits(C[mt][nt][i]);
      }
    }
}

template <int PATH, int FMT, int GPT>
int launch_f16(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
               const uint16_t* zero, uint16_t* y, hipStream_t s) {
  if ((size_t)M * K * 2 >= (1ull << 32))
    return fail(-2 /* W4_EUNSUPPORTED */, "w4_gemm: activations of %d x %d exceed the 4 GiB one call addresses", M, K);
  static bool attr_set = false;  // one-time opt-in to more than 64 KB of LDS
  if (!attr_set) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_f16_kernel<PATH, FMT, GPT>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, 2 * kF16Stage);
    if (e != hipSuccess) return fail(-4 /* W4_EHIP */, "w4_gemm: cannot reserve %d bytes of LDS: %s", 2 * kF16Stage,
                                     hipGetErrorString(e));
    attr_set = true;
  }
  const long tiles = (long)((N + kF16BN - 1) / kF16BN) * ((M + kF16BM - 1) / kF16BM);
  hipLaunchKernelGGL((gemm_f16_kernel<PATH, FMT, GPT>), dim3((unsigned)tiles), dim3(kF16Threads), 2 * kF16Stage, s, x,
                     M, K, N, packed, scale, zero, y);
  return check_launch("gemm");
}

template <int PATH, int FMT, int GPT, int NT, int NS>
int launch_one(const void* a, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
               const uint16_t* zero, uint16_t* y, const float* tok_scale, const int32_t* gsum, int32_t* acc_out,
               hipStream_t s) {
  using Geo = GemmGeom<PATH, NT, NS, GPT>;
  static_assert(Geo::A_UNITS % kGemmThreads == 0, "activation tile must split evenly over the threads");
  static_assert(GPT * Geo::BN <= kGemmThreads && GPT * kBM <= kGemmThreads, "one scale / row sum per thread");
  const long tiles = (long)((N + Geo::BN - 1) / Geo::BN) * ((M + kBM - 1) / kBM);
  if (acc_out)
    hipLaunchKernelGGL((gemm_kernel<PATH, FMT, GPT, NT, NS, true>), dim3((unsigned)tiles), dim3(kGemmThreads), Geo::LDS,
                       s, a, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out);
  else
    hipLaunchKernelGGL((gemm_kernel<PATH, FMT, GPT, NT, NS, false>), dim3((unsigned)tiles), dim3(kGemmThreads),
                       Geo::LDS, s, a, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out);
  return check_launch(PATH == 2 ? "gemm_msd" : "gemm");
}

}  // namespace

int launch_gemm(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                const uint16_t* zero, int G, int fmt, int mode, uint16_t* y, hipStream_t s) {
#define W4_GEMM_CASE(PATH, FMT, GPT) return launch_f16<PATH, FMT, GPT>(x, M, K, N, packed, scale, zero, y, s)
  if (mode == 0) {
    if (fmt == 0) {
      if (G == 64) W4_GEMM_CASE(0, 0, 2);
      W4_GEMM_CASE(0, 0, 1);
    }
    if (G == 64) W4_GEMM_CASE(0, 1, 2);
    W4_GEMM_CASE(0, 1, 1);
  }
  if (fmt == 0) {
    if (G == 64) W4_GEMM_CASE(1, 0, 2);
    W4_GEMM_CASE(1, 0, 1);
  }
  if (G == 64) W4_GEMM_CASE(1, 1, 2);
  W4_GEMM_CASE(1, 1, 1);
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
    if (G == 64) return launch_one<2, 0, 2, NT, 1>(slices, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out, s);
    return launch_one<2, 0, 1, NT, 1>(slices, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out, s);
  }
  if (G == 64) return launch_one<2, 0, 2, NT, 2>(slices, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out, s);
  return launch_one<2, 0, 1, NT, 2>(slices, M, K, N, packed, scale, zero, y, tok_scale, gsum, acc_out, s);
}

}  // namespace w4

// MXFP4 weights and the two-pass MXFP4 decomposition of the activations on
// the block-scaled fp4 matrix cores ("Multi-Scale Dequant: Eliminating
// Dequantization Bottleneck via Activation Decomposition for Efficient LLM
// Inference", Abstract: MXFP4 weights, activations split into two MXFP4
// parts, each multiplied with the weights directly).
//
// MXFP4 (the published OCP Microscaling format): 4-bit E2M1 elements (sign,
// 2-bit exponent with bias 1, 1-bit mantissa: magnitudes 0, 0.5, 1, 1.5, 2, 3,
// 4, 6) and one E8M0 scale 2^(s - 127) per 32 consecutive K positions.  Scale
// rule (a reading; the pages give none): the smallest e with amax <= 6 * 2^e,
// so no element saturates.  Rounding to E2M1 is to nearest, ties to the even
// mantissa; a zero result carries no sign.  The scaled values and residuals
// are exact (see below), so every decision is the exact one.
//
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 with fp4 operands takes, per
// lane l, 16 bytes of A (row l % 16, K positions 32 (l / 16) .. + 31, two per
// byte, low nibble first), the same for B (column l % 16), and one E8M0 byte
// per operand for that lane's 32 positions; it applies both scales itself.
// So a slice row stored as plain packed nibbles is already in operand order,
// and the product needs no per-group epilogue: both slices accumulate into
// the same fp32 tile.
#include "w4_device.h"
#include "w4_internal.h"

#include <cstdlib>

#pragma clang fp contract(off)

namespace w4 {
namespace {

constexpr int kMxBlock = 32;
constexpr int kMxStepK = 128;

typedef int v8i __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- encoding
// All arithmetic below is exact in fp32 for fp16 or fp32 inputs and up to two
// passes: scaling by a power of two is exact (no overflow: |v| / 2^e <= 6;
// no underflow for the values that occur), and a first-pass residual
// v - q 2^e needs at most 13 significant bits (|v| >= 2^(e-2) when q != 0,
// so v's last bit is at least 2^(e-12), and |v - q 2^e| <= 2^e).  The
// decisions therefore match an fp64 evaluation bit for bit.

// smallest e with amax <= 6 * 2^e: with amax = f 2^p, f in [0.5, 1), it is
// p - 3 when f <= 0.75 and p - 2 otherwise
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  int p;
  const float f = frexpf(amax, &p);
  const int e = f <= 0.75f ? p - 3 : p - 2;
  return min(max(e, -127), 127);
}

// E2M1 code of t (round to nearest, ties to even, |t| saturated at 6),
// without branches: below 1 the code is rint(2 |t|) (0, 0.5 or 1.0); from 1
// on, |t| rounded to one mantissa bit on its fp32 bit pattern is (1 + m/2) 2^E
// and the code is 2 E + 2 + m.
__device__ __forceinline__ int e2m1_code(float t) {
  const float a = fminf(fabsf(t), 6.f);
  const int lo = (int)__builtin_rintf(2.f * a);
  const uint32_t b = __float_as_uint(a);
  const uint32_t r = b + 0x1FFFFFu + ((b >> 22) & 1u);  // carry into the exponent allowed
  const int hi = (int)(r >> 22) - 2 * 127 + 2;             // 2 (E + 127) + m - 254 + 2
  const int c = a < 1.f ? lo : hi;
  return (t < 0.f && c != 0) ? (c | 8) : c;
}

// magnitude of code c (0..7): 0.5 c below 2, else (1 + m/2) 2^(c/2 - 1)
__device__ __forceinline__ float e2m1_mag(int c) {
  const float big = __uint_as_float(((uint32_t)((c >> 1) + 126) << 23) | ((uint32_t)(c & 1) << 22));
  return c < 2 ? 0.5f * (float)c : big;
}

// one 32-element block: codes and exponent of v (v is left as the residual)
__device__ __forceinline__ int mx_block(float (&v)[kMxBlock], uint8_t (&code)[kMxBlock]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int e = mx_exponent(amax);
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) {
    const int c = e2m1_code(ldexpf(v[i], -e));
    code[i] = (uint8_t)c;
    const float q = ldexpf(e2m1_mag(c & 7), e);
    v[i] = v[i] - ((c & 8) ? -q : q);
  }
  return e;
}

__device__ __forceinline__ u32x4 pack_nibbles(const uint8_t (&code)[kMxBlock]) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t x = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) x |= (uint32_t)code[8 * q + i] << (4 * i);
    w[q] = x;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// ------------------------------------------------------- weight quantizer
// One thread per (row, block of 32): codes (one per byte) and E8M0 scales.
__global__ __launch_bounds__(256) void quantize_mx_kernel(const float* __restrict__ wt, int K, int N,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scale) {
  const int nb = K / kMxBlock;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long)N * nb) return;
  const long n = t / nb, b = t % nb;
  const float* src = wt + n * K + b * kMxBlock;
  float v[kMxBlock];
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) v[i] = src[i];
  uint8_t c[kMxBlock];
  const int e = mx_block(v, c);
  uint8_t* dst = codes + n * K + b * kMxBlock;
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) dst[i] = c[i];
  scale[n * nb + b] = (uint8_t)(e + 127);
}

// codes [N][K] -> 1 KB tiles (16 rows x 128 K positions); lane l = 16 j + r of
// a tile holds row r's positions 32 j .. 32 j + 31, two per byte, low first.
__global__ __launch_bounds__(256) void pack_mx_kernel(const uint8_t* __restrict__ codes, int K, int N,
                                                      uint8_t* __restrict__ packed) {
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;  // one 16-byte piece
  const long KT = K / kMxStepK;
  if (t >= (long)(N / 16) * KT * 64) return;
  const long tile = t / 64;
  const int l = (int)(t % 64), j = l / 16, r = l % 16;
  const long nb = tile / KT, kb = tile % KT;
  const uint8_t* src = codes + (nb * 16 + r) * K + kb * kMxStepK + 32 * j;
  uint8_t c[kMxBlock];
#pragma unroll
  for (int i = 0; i < kMxBlock; ++i) c[i] = src[i];
  *reinterpret_cast<u32x4*>(packed + t * 16) = pack_nibbles(c);
}

// ------------------------------------------------- activation decomposition
// One thread per (token, block of 32): NS passes, each the MXFP4 of the
// residual the earlier passes left.  Slices [NS][M][K/2] (packed nibbles,
// low first) and E8M0 scales [NS][M][K/32].
template <int NS>
__global__ __launch_bounds__(256) void decompose_mx_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                           uint8_t* __restrict__ slices, uint8_t* __restrict__ scales,
                                                           uint8_t* __restrict__ slices_out,
                                                           uint8_t* __restrict__ scales_out) {
  const int nb = K / kMxBlock;
  const long t = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (long)M * nb) return;
  const long m = t / nb, b = t % nb;
  const u32x4* src = reinterpret_cast<const u32x4*>(x + m * K + b * kMxBlock);
  float v[kMxBlock];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4 w = src[q];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[8 * q + 2 * i] = half_bits_to_float((uint16_t)(w[i] & 0xFFFFu));
      v[8 * q + 2 * i + 1] = half_bits_to_float((uint16_t)(w[i] >> 16));
    }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    uint8_t c[kMxBlock];
    const int e = mx_block(v, c);
    const u32x4 p = pack_nibbles(c);
    const size_t row = (size_t)j * M + m;
    *reinterpret_cast<u32x4*>(slices + row * (K / 2) + b * 16) = p;
    scales[row * nb + b] = (uint8_t)(e + 127);
    if (slices_out) *reinterpret_cast<u32x4*>(slices_out + row * (K / 2) + b * 16) = p;
    if (scales_out) scales_out[row * nb + b] = (uint8_t)(e + 127);
  }
}

// ------------------------------------------------------------------ product
// Workgroups of 8 waves own (128 WM) tokens x 256 weight rows; the waves form
// a WM x (8 / WM) grid, each 128 x (32 WM) (8 x 2 WM products of 16 x 16 per
// slice), so each activation operand read from LDS serves 2 WM products.
// WM = 2 halves the activation reads per product; WM = 1 makes twice as many,
// smaller tiles (more even filling of the GPU).  K step 128 (one block-scaled product per tile pair),
// three stages of global -> LDS copies:
//  * slice j's step tile: 128 WM rows x 64 bytes; 16-byte chunk c of row m
//    sits at chunk c ^ ((m >> 2) & 3), so the 16 lanes reading one chunk
//    column of 16 rows hit 16 different bank groups;
//  * the 16 weight tiles of the step (1 KB each, lane l's operand at 16 l);
//  * the step's E8M0 bytes as 4-byte words: [slice][row] and [column], each
//    word the row's (column's) four blocks of the step; a lane extracts its
//    own block's byte.
constexpr int kMxThreads = 512;
constexpr int kMxBN = 256;
constexpr int kMxB = (kMxBN / 16) * 1024;
constexpr int kMxSB = kMxBN * 4;
constexpr int kMxStages = 3;
template <int WM>
constexpr int mx_bm() { return 128 * WM; }
template <int NS, int WM>
constexpr int mx_stage_bytes() { return NS * mx_bm<WM>() * 64 + kMxB + NS * mx_bm<WM>() * 4 + kMxSB; }
// waves along M (measured at M = 2048, K = 5120, N = 25600: WM = 2 is faster
// for one slice, 226 vs 286 us, and for two, 437 vs 450 us)
template <int NS>
constexpr int mx_wm() { return 2; }

__device__ __forceinline__ f32x4 mfma_fp4(u32x4 a, uint32_t sa, u32x4 b, uint32_t sb, f32x4 c) {
  const v8i av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  const v8i bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

template <int NS, int WM>
__global__ __launch_bounds__(kMxThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_mx_kernel(
    const uint8_t* __restrict__ slices, const uint8_t* __restrict__ xscale, int M, int K, int N,
    const uint8_t* __restrict__ packed, const uint8_t* __restrict__ wscale, uint16_t* __restrict__ y,
    float* __restrict__ tpart, int tile0, int gm) {
  constexpr int BM = mx_bm<WM>();
  constexpr int WN = 8 / WM;                // waves along N
  constexpr int MT = 8, NT = 2 * WM;
  constexpr int kA = BM * 64, kSA = BM * 4;
  constexpr int kStage = mx_stage_bytes<NS, WM>();
  constexpr int kOffB = NS * kA, kOffSA = kOffB + kMxB, kOffSB = kOffSA + NS * kSA;
  constexpr int kScaleCopies = NS * (BM / 64) + 4;  // 64 rows or columns each
  constexpr int kScW = (kScaleCopies + 7) / 8;      // per wave (the last repeat earlier ones)
  constexpr int kCopies = NS * WM + 2 + kScW;       // per wave per step
  static_assert(kCopies < 16, "copy count must fit the low vmcnt field");
  extern __shared__ __align__(16) unsigned char smem[];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wn = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wn / WN, wc = wn % WN;  // this wave: rows 128 wm .., columns 16 NT wc ..
  const int ln = lane % 16, jb = lane / 16;

  const int tiles_n = (N + kMxBN - 1) / kMxBN;
  const int place = tile0 + xcd_run(blockIdx.x, gridDim.x);
  int mb, nb;
  tile_mn(place, (M + BM - 1) / BM, tiles_n, gm, mb, nb);
  const int n0 = nb * kMxBN;
  const int m0 = mb * BM;

  const int KT = K / kMxStepK;
  // K slice (gridDim.y > 1 only for a tail launch, whose partials go to tpart)
  const int S = gridDim.y, ks = blockIdx.y;
  const int kt0 = (int)((long)KT * ks / S), kt1 = (int)((long)KT * (ks + 1) / S);
  const int nbk = K / kMxBlock;  // scale bytes per row
  const int ntile_last = N / 16 - 1;

  // descriptors from scalar sizes (each slice and its scales on their own,
  // so rows past M read zeros)
  const uint32_t slice_bytes = __builtin_amdgcn_readfirstlane((uint32_t)M * (uint32_t)(K / 2));
  const uint32_t xs_bytes = __builtin_amdgcn_readfirstlane((uint32_t)M * (uint32_t)nbk);
  auto ar = [&](int j) { return make_rsrc(slices + (size_t)j * slice_bytes, slice_bytes); };
  auto sr = [&](int j) { return make_rsrc(xscale + (size_t)j * xs_bytes, xs_bytes); };
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(packed, (uint32_t)((size_t)N * (K / 2)));
  const __amdgpu_buffer_rsrc_t wsr = make_rsrc(wscale, (uint32_t)((size_t)N * nbk));

  // wave wn copies rows 16 WM wn + 16 i .. + 15 (i < WM) of each slice: lane l
  // -> row + l / 4, LDS chunk l % 4, which holds global chunk (l % 4) ^ ((l / 16) & 3)
  uint32_t voff_a[WM];
#pragma unroll
  for (int i = 0; i < WM; ++i)
    voff_a[i] = (uint32_t)(m0 + 16 * WM * wn + 16 * i + lane / 4) * (uint32_t)(K / 2) +
                (uint32_t)(((lane % 4) ^ ((lane / 16) & 3)) * 16);
  uint32_t voff_b[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    voff_b[j] = (uint32_t)min(n0 / 16 + 2 * wn + j, ntile_last) * (uint32_t)KT * 1024 + (uint32_t)lane * 16;
  // scale copies: c < NS BM/64: slice c / (BM/64), rows 64 (c % (BM/64)) +
  // lane; otherwise columns 64 (c - NS BM/64) + lane
  constexpr int kRowSc = BM / 64;
  uint32_t voff_s[kScW];
  int sc_dst[kScW];
  bool sc_x[kScW];
  int sc_j[kScW];
#pragma unroll
  for (int i = 0; i < kScW; ++i) {
    const int c = (wn * kScW + i) % kScaleCopies;
    sc_x[i] = c < NS * kRowSc;
    sc_j[i] = sc_x[i] ? c / kRowSc : 0;
    voff_s[i] = sc_x[i] ? (uint32_t)(m0 + 64 * (c % kRowSc) + lane) * (uint32_t)nbk
                        : (uint32_t)(n0 + 64 * (c - NS * kRowSc) + lane) * (uint32_t)nbk;
    sc_dst[i] = sc_x[i] ? kOffSA + sc_j[i] * kSA + 64 * (c % kRowSc) * 4 : kOffSB + 64 * (c - NS * kRowSc) * 4;
  }

  auto stage = [&](int kt) { return smem + ((kt - kt0) % kMxStages) * kStage; };
  auto issue_step = [&](int kt) {
    unsigned char* st = stage(kt);
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < WM; ++i)
        copy16_to_lds(ar(j), voff_a[i], (uint32_t)kt * 64, st + j * kA + (16 * WM * wn + 16 * i) * 64);
#pragma unroll
    for (int j = 0; j < 2; ++j) copy16_to_lds(wr, voff_b[j], (uint32_t)kt * 1024, st + kOffB + (2 * wn + j) * 1024);
#pragma unroll
    for (int i = 0; i < kScW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(sc_x[i] ? sr(sc_j[i]) : wsr, (lds_void*)(st + sc_dst[i]), 4, voff_s[i],
                                               (uint32_t)kt * 4, 0, 0);
  };
  auto wait_all_but_one_step = [&]() { __builtin_amdgcn_s_waitcnt(kCopies | (0x7 << 4) | (0xF << 8)); };

  f32x4 C[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) C[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const uint32_t a_chunk = (uint32_t)((jb ^ ((ln >> 2) & 3)) * 16);
  const uint32_t shift = 8u * (uint32_t)jb;

  issue_step(kt0);
  if (kt1 - kt0 > 1) {
    issue_step(kt0 + 1);
    wait_all_but_one_step();
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const unsigned char* cur = stage(kt);
    const bool more2 = kt + 2 < kt1;
    if (more2) issue_step(kt + 2);

    u32x4 Bv[NT];
    uint32_t sb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      Bv[nt] = *reinterpret_cast<const u32x4*>(cur + kOffB + (NT * wc + nt) * 1024 + lane * 16);
      sb[nt] = __builtin_amdgcn_ubfe(
          *reinterpret_cast<const uint32_t*>(cur + kOffSB + (wc * 16 * NT + nt * 16 + ln) * 4), shift, 8);
    }
    // slice fragments and scales of token tile mt; tile mt + 1's are read
    // before tile mt's products run
    u32x4 Af[2][NS];
    uint32_t saf[2][NS];
    auto load_frag = [&](int b, int mt) {
      const int row = wm * 128 + mt * 16 + ln;
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        Af[b][j] = *reinterpret_cast<const u32x4*>(cur + j * kA + row * 64 + a_chunk);
        saf[b][j] = *reinterpret_cast<const uint32_t*>(cur + kOffSA + j * kSA + row * 4);
      }
    };
    load_frag(0, 0);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      if (mt + 1 < MT) load_frag((mt + 1) % 2, mt + 1);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const uint32_t sa = __builtin_amdgcn_ubfe(saf[mt % 2][j], shift, 8);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) C[mt][nt] = mfma_fp4(Af[mt % 2][j], sa, Bv[nt], sb[nt], C[mt][nt]);
      }
    }

    if (more2)
      wait_all_but_one_step();  // step kt+1's copies have landed
    else
      __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();  // everyone's have, and nobody still reads this step's buffer
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + wm * 128 + mt * 16 + 4 * jb + i;
      if (m >= M) continue;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + wc * 16 * NT + nt * 16 + ln;
        if (n >= N) continue;
        if (tpart)
          tpart[(((size_t)ks * gridDim.x + (place - tile0)) * BM + (m - m0)) * kMxBN + (n - n0)] = C[mt][nt][i];
        else
          y[(size_t)m * N + n] = float_to_half_bits(C[mt][nt][i]);
      }
    }
}

template <int NS, int WM>
int launch_gemm_mx_w(const uint8_t* slices, const uint8_t* xscale, int M, int K, int N, const uint8_t* packed,
                     const uint8_t* wscale, uint16_t* y, float* tpart, size_t tpart_bytes, hipStream_t s) {
  constexpr int kLds = kMxStages * mx_stage_bytes<NS, WM>();
  constexpr int BM = mx_bm<WM>();
  static_assert(kLds <= 160 * 1024, "LDS");
  const int st = allow_dynamic_lds(reinterpret_cast<const void*>(&gemm_mx_kernel<NS, WM>), kLds, "w4_gemm_mx");
  if (st != 0) return st;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + kMxBN - 1) / kMxBN;
  const long tiles = (long)tiles_n * tiles_m;
  const int gm = gemm_group_rows();
  const TailPlan tp = plan_tail(tiles, K / kMxStepK, BM, kMxBN);
  const bool tail = tp.S > 1 && tpart && tpart_bytes >= tp.bytes;
  const long main_tiles = tail ? tp.main : tiles;
  int st2;
  if (main_tiles > 0) {
    hipLaunchKernelGGL((gemm_mx_kernel<NS, WM>), dim3((unsigned)main_tiles), dim3(kMxThreads), kLds, s, slices,
                       xscale, M, K, N, packed, wscale, y, nullptr, 0, gm);
    if ((st2 = check_launch("gemm_mx")) != 0) return st2;
  }
  if (!tail) return 0;
  hipLaunchKernelGGL((gemm_mx_kernel<NS, WM>), dim3((unsigned)tp.r, (unsigned)tp.S), dim3(kMxThreads), kLds, s,
                     slices, xscale, M, K, N, packed, wscale, y, tpart, (int)tp.main, gm);
  if ((st2 = check_launch("gemm_mx tail")) != 0) return st2;
  return launch_tail_reduce(tpart, tp, BM, kMxBN, tiles_m, tiles_n, gm, M, N, y, s);
}

// waves along M of the MXFP4 product with ns slices (W4_MX_WM = 1 or 2
// overrides it for sweeps)
int mx_wm_for(int ns) {
  static const int wm = [] {
    const char* e = std::getenv("W4_MX_WM");
    return e && (*e == '1' || *e == '2') ? *e - '0' : 0;
  }();
  if (wm) return wm;
  return ns == 1 ? mx_wm<1>() : mx_wm<2>();
}

template <int NS>
int launch_gemm_mx_t(const uint8_t* slices, const uint8_t* xscale, int M, int K, int N, const uint8_t* packed,
                     const uint8_t* wscale, uint16_t* y, float* tpart, size_t tpart_bytes, hipStream_t s) {
  if (mx_wm_for(NS) == 1)
    return launch_gemm_mx_w<NS, 1>(slices, xscale, M, K, N, packed, wscale, y, tpart, tpart_bytes, s);
  return launch_gemm_mx_w<NS, 2>(slices, xscale, M, K, N, packed, wscale, y, tpart, tpart_bytes, s);
}

inline unsigned blocks_for(long threads) { return (unsigned)((threads + 255) / 256); }

}  // namespace

int launch_quantize_mx(const float* wt, int K, int N, uint8_t* codes, uint8_t* scale, hipStream_t s) {
  hipLaunchKernelGGL(quantize_mx_kernel, dim3(blocks_for((long)N * (K / kMxBlock))), dim3(256), 0, s, wt, K, N,
                     codes, scale);
  return check_launch("quantize_mx");
}

int launch_pack_mx(const uint8_t* codes, int K, int N, uint8_t* packed, hipStream_t s) {
  hipLaunchKernelGGL(pack_mx_kernel, dim3(blocks_for((long)(N / 16) * (K / kMxStepK) * 64)), dim3(256), 0, s, codes,
                     K, N, packed);
  return check_launch("pack_mx");
}

size_t mx_workspace_bytes(int M, int K, int nslices) {
  const size_t sl = ((size_t)nslices * M * (K / 2) + 255) / 256 * 256;
  const size_t sc = ((size_t)nslices * M * (K / kMxBlock) + 255) / 256 * 256;
  return sl + sc;
}

size_t mx_tail_bytes(int M, int K, int N, int nslices) {
  const int bm = 128 * mx_wm_for(nslices);
  const long tiles = (long)((N + kMxBN - 1) / kMxBN) * ((M + bm - 1) / bm);
  return plan_tail(tiles, K / kMxStepK, bm, kMxBN).bytes;
}

int launch_gemm_mx(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint8_t* wscale, int nslices,
                   uint16_t* y, uint8_t* slices_out, uint8_t* scales_out, void* ws, size_t ws_bytes, hipStream_t s) {
  uint8_t* sl = static_cast<uint8_t*>(ws);
  uint8_t* sc = sl + ((size_t)nslices * M * (K / 2) + 255) / 256 * 256;
  const unsigned blocks = blocks_for((long)M * (K / kMxBlock));
  if (nslices == 1)
    hipLaunchKernelGGL(decompose_mx_kernel<1>, dim3(blocks), dim3(256), 0, s, x, M, K, sl, sc, slices_out,
                       scales_out);
  else
    hipLaunchKernelGGL(decompose_mx_kernel<2>, dim3(blocks), dim3(256), 0, s, x, M, K, sl, sc, slices_out,
                       scales_out);
  const int st = check_launch("decompose_mx");
  if (st != 0) return st;
  // the tail's partials, when the workspace holds them after the slices and scales
  const size_t base = mx_workspace_bytes(M, K, nslices);
  float* tpart = ws_bytes > base ? reinterpret_cast<float*>(static_cast<char*>(ws) + base) : nullptr;
  const size_t tbytes = ws_bytes > base ? ws_bytes - base : 0;
  if (nslices == 1) return launch_gemm_mx_t<1>(sl, sc, M, K, N, packed, wscale, y, tpart, tbytes, s);
  return launch_gemm_mx_t<2>(sl, sc, M, K, N, packed, wscale, y, tpart, tbytes, s);
}

}  // namespace w4

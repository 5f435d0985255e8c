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
//           Hardware Co-design for Efficient LLM Inference", Abstract: the
//           dequantization moves after the per-group product).
//  PATH_MSD Multi-Scale Dequant: the activations arrive as int8 slices; the
//           4-bit codes are widened to int8 with mask/shift only (no
//           conversion to a floating type) and meet every slice on the int8
//           matrix cores, the same weight operand serving both slices; group
//           scales, zero points and token scales are applied after the
//           integer accumulation of each group.
//
// Tiling.  Workgroups of 8 waves (two per SIMD: one wave alone cannot keep a
// matrix core busy) own 256 tokens x 128 weight rows (fp16 paths) or 128 x
// 128 (MSD).  The K loop steps one weight-tile column (128 K positions: one
// or two quantization groups) at a time.  Each step's activation tile,
// weight tiles and scales are copied global -> LDS by the load unit itself,
// double buffered, with one barrier per step.
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

#include <algorithm>
#include <atomic>
#include <cstdlib>

namespace w4 {
namespace {

constexpr int kStepK = 128;  // one weight-tile column per K step

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pk_sub_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) - __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// ---------------------------------------------------------------------------
// Both matrix-core kernels run 8 waves per workgroup, two per SIMD (one wave
// alone cannot keep a matrix core busy), one workgroup per CU.  Operand tiles
// are copied global -> LDS by the load unit itself (16 bytes per lane, lane
// l's bytes landing at the instruction's LDS base + 16 l).  In LDS, a token
// row's 16-byte chunk c sits at c ^ (row mod 16) (fp16) or c ^ (row mod 8)
// (int8), which keeps both the fill and the operand reads free of bank
// conflicts.
constexpr int kF16Threads = 512;  // 8 waves


// fp16 paths: 128 tokens x 256 weight rows per workgroup, the 8 waves side by
// side along N (each 128 x 32: 8 x 2 products of 16 x 16), so every weight
// operand is unpacked by exactly one wave and serves 128 token rows.  A K step
// moves 32 KB of activations, 16 KB of weight tiles and the scales -- a third
// fewer bytes per product than a 256 x 128 block -- and the 50 KB stage allows
// three buffers: steps k+1 and k+2 are in flight while step k is computed.
// The scales (and zero points) of a step travel the same way: a 2-byte copy
// puts lane l's value, zero-extended, in the dword at base + 4 l, so a step's
// scales land as [group][scale, zero][256] dwords; their load latency hides
// behind two steps like the tiles' (a plain load consumed within its step
// exposed one memory latency per step).
constexpr int kHBM = 128;
constexpr int kHBN = 256;
constexpr int kHA = kHBM * 256;          // activation tile bytes per stage
constexpr int kHB = (kHBN / 16) * 1024;  // weight tiles
constexpr int kHS = 2 * 2 * kHBN * 4;    // [group in step][scale, zero][BN] dwords
constexpr int kHStage = kHA + kHB + kHS;
constexpr int kHStages = 3;
constexpr int kHTileCopies = kHA / (kF16Threads * 16) + kHB / (kF16Threads * 16);  // per wave per step
// scale copies per wave per step: GPT groups x (scale [, zero]) x 4 x 64 columns over 8 waves
constexpr int h_scale_copies(int fmt, int gpt) { return (gpt * (fmt == 0 ? 2 : 1) * 4 + 7) / 8; }

template <int PATH, int FMT, int GPT>
__global__ __launch_bounds__(kF16Threads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_f16_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    float* __restrict__ partial, float* __restrict__ tpart, int tile0, int gm) {
  constexpr int G = kStepK / GPT;
  constexpr int WPG = 4 / GPT;  // products (tile words) per group
  constexpr int MT = 8, NT = 2;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wn = __builtin_amdgcn_readfirstlane(tid / kWave);  // the wave: columns 32 wn .. 32 wn + 31
  const int S = gridDim.y;  // K slices (partials in `partial`, or `tpart` for a tail launch, when S > 1)
  const int ks = blockIdx.y;
  const int ln = lane % 16, kb = lane / 16;

  // XCD-aware, row-block-grouped renumbering (a bijection of the launch's
  // places [tile0, tile0 + gridDim.x) of the walk)
  const int tiles_n = (N + kHBN - 1) / kHBN;
  const int place = tile0 + xcd_run(blockIdx.x, gridDim.x);
  int mb, nb;
  tile_mn(place, (M + kHBM - 1) / kHBM, tiles_n, gm, mb, nb);
  const int n0 = nb * kHBN;
  const int m0 = mb * kHBM;

  const int ng = K / G;
  const int KT = K / kStepK;
  const int ntile_last = N / 16 - 1;
  const int kt0 = (int)((long)KT * ks / S), kt1 = (int)((long)KT * (ks + 1) / S);  // this slice's steps

  if constexpr (FMT == 1) {
    for (int i = tid; i < 256; i += kF16Threads)
      lut[i] = (uint32_t)float_to_half_bits(nf4_level(i & 15)) |
               ((uint32_t)float_to_half_bits(nf4_level(i >> 4)) << 16);
  }

  // ---- per-lane copy offsets (fixed for the whole K loop; the step adds a
  // scalar offset).  Wave w fills token rows [16 w, 16 w + 16), 4 rows per
  // instruction, and weight tiles 2 w and 2 w + 1.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(packed, (uint32_t)((size_t)N * (K / 2)));
  uint32_t voff_a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = wn * 16 + 4 * i + lane / 16;
    const int c = (lane % 16) ^ (row & 15);
    voff_a[i] = (uint32_t)(m0 + row) * (uint32_t)(K * 2) + (uint32_t)c * 16;  // rows past M read zeros
  }
  uint32_t voff_b[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    voff_b[j] = (uint32_t)min(n0 / 16 + 2 * wn + j, ntile_last) * (uint32_t)KT * 1024 + (uint32_t)lane * 16;
  // scale copies: instruction c (of GPT x arrays x 4) covers group c / (4 A),
  // array (c / 4) % A (0 scale, 1 zero), columns 64 (c % 4) .. + 63; every
  // wave issues kSC of them (the last ones repeat earlier ones when the count
  // does not divide: identical bytes to identical places), so that every wave
  // has the same number of copies in flight
  constexpr int kArrays = FMT == 0 ? 2 : 1;
  constexpr int kSCTotal = GPT * kArrays * 4;
  constexpr int kSC = h_scale_copies(FMT, GPT);
  constexpr int kCopies = kHTileCopies + kSC;
  static_assert(kCopies < 16, "copy count must fit the low vmcnt field");
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scale, (uint32_t)((size_t)N * ng * 2));
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(FMT == 0 ? zero : scale, (uint32_t)((size_t)N * ng * 2));
  uint32_t voff_s[kSC];
  int sc_dst[kSC];
#pragma unroll
  for (int j = 0; j < kSC; ++j) {
    const int c = (wn * kSC + j) % kSCTotal;
    const int gi = c / (4 * kArrays), arr = (c / 4) % kArrays, quarter = c % 4;
    const int col = quarter * 64 + lane;
    // columns past N read zeros (the buffer's range check)
    voff_s[j] = (uint32_t)(n0 + col) * (uint32_t)ng * 2u + (uint32_t)gi * 2u;
    sc_dst[j] = kHA + kHB + ((gi * 2 + arr) * kHBN + quarter * 64) * 4;
  }
  auto stage = [&](int kt) { return smem + ((kt - kt0) % kHStages) * kHStage; };
  auto issue_step = [&](int kt) {
    unsigned char* st = stage(kt);
#pragma unroll
    for (int i = 0; i < 4; ++i) copy16_to_lds(xr, voff_a[i], (uint32_t)kt * 256, st + (wn * 16 + 4 * i) * 256);
#pragma unroll
    for (int j = 0; j < 2; ++j) copy16_to_lds(wr, voff_b[j], (uint32_t)kt * 1024, st + kHA + (2 * wn + j) * 1024);
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      const int c = (wn * kSC + j) % kSCTotal;
      const __amdgpu_buffer_rsrc_t rr = ((c / 4) % kArrays) == 1 ? zr : sr;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rr, (lds_void*)(st + sc_dst[j]), 2, voff_s[j], (uint32_t)kt * GPT * 2u,
                                               0, 0);
    }
  };
  // all but the newest step's copies have landed (vmcnt = kCopies in the low
  // field, bits 15:14 zero; expcnt and lgkmcnt left at their maxima)
  auto wait_all_but_one_step = [&]() { __builtin_amdgcn_s_waitcnt(kCopies | (0x7 << 4) | (0xF << 8)); };
  // operand-read offsets within a stage: word w of token tile mt at
  // a_off[w] + mt * 4096 (swizzled chunk 4w + kb of row mt*16 + ln)
  uint32_t a_off[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) a_off[w] = (uint32_t)ln * 256 + ((uint32_t)((4 * w + kb) ^ ln) << 4);

  f32x4 C[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) C[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // ---- prologue: the slice's first two steps in flight, the first landed
  issue_step(kt0);
  if (kt1 - kt0 > 1) {
    issue_step(kt0 + 1);
    wait_all_but_one_step();
  } else {
    __builtin_amdgcn_s_waitcnt(0);
  }
  __syncthreads();

  // DQ, INT4: the nibble mask held in a VGPR (opaque to the compiler), so that
  // (v >> 4j) & mask | 0x64006400 is one v_and_or_b32 with the constant in an
  // SGPR (one constant-bus operand) instead of a separate and and or
  uint32_t nib_mask = 0x000F000Fu;
  if constexpr (PATH == 0 && FMT == 0) asm volatile("v_mov_b32 %0, 0x000F000F" : "=v"(nib_mask));

  // per-step state: raw weight words, per-column scales / zero points
  u32x4 Bq[NT];
  float sfv[GPT][NT];      // PS: per-column scale (x 2^24 for INT4)
  uint32_t zzv[GPT][NT];   // INT4: zero-point pair
  uint32_t spv[GPT][NT];   // DQ: (s, s) pair
  auto load_step = [&](const unsigned char* cur) {
    const uint32_t* s_lds = reinterpret_cast<const uint32_t*>(cur + kHA + kHB);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Bq[nt] = *reinterpret_cast<const u32x4*>(cur + kHA + (2 * wn + nt) * 1024 + lane * 16);
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = wn * 32 + nt * 16 + ln;
        const uint32_t sb = s_lds[(gi * 2) * kHBN + col];
        spv[gi][nt] = sb | (sb << 16);
        sfv[gi][nt] = half_bits_to_float((uint16_t)sb) * (FMT == 0 ? 16777216.0f : 1.0f);
        zzv[gi][nt] = 0;
        if constexpr (FMT == 0) {
          const uint32_t z = (uint32_t)half_bits_to_float(s_lds[(gi * 2 + 1) * kHBN + col]);  // 0..15
          // PS: (z, z) * 2^-24 as subnormal fp16; DQ: (1024 + z, 1024 + z)
          zzv[gi][nt] = PATH == 1 ? (z | (z << 16)) : ((0x6400u | z) | ((0x6400u | z) << 16));
        }
      }
  };
  auto unpack = [&](u32x4 (&Bu)[NT], int w) {
    const int gi = w / WPG;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint32_t v = Bq[nt][w];
      if constexpr (FMT == 0) {
        uint32_t d[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint32_t q = (v >> (4 * j)) & nib_mask;  // (c_2j, c_2j+1) * 2^-24
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
  auto load_a = [&](const unsigned char* cur, u32x4 (&A)[MT], int w) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) A[mt] = *reinterpret_cast<const u32x4*>(cur + a_off[w] + mt * 4096);
  };
  f32x4 acc[MT][NT];  // PS: the group's partial products
  // one word's 16 products (PS: into the group's partial products)
  auto products = [&](const u32x4 (&A)[MT], const u32x4 (&Bc)[NT], int w) {
    const bool first = (w % WPG) == 0;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if constexpr (PATH == 1) acc[mt][nt] = mfma_f16(A[mt], Bc[nt], first ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[mt][nt]);
        else C[mt][nt] = mfma_f16(A[mt], Bc[nt], C[mt][nt]);
      }
  };
  // PS: a group is complete; scale its partial products once
  auto scale_group = [&](int gi) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i) C[mt][nt][i] = fmaf(sfv[gi][nt], acc[mt][nt][i], C[mt][nt][i]);
  };

  for (int kt = kt0; kt < kt1; ++kt) {
    const unsigned char* cur = stage(kt);
    const bool more2 = kt + 2 < kt1;
    if (more2) issue_step(kt + 2);
    load_step(cur);

    // Word by word, the next word's operands are read and unpacked while this
    // word's 16 products run.
    u32x4 B0[NT], B1[NT];
    u32x4 A0[MT], A1[MT];
    load_a(cur, A0, 0);
    unpack(B0, 0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      u32x4(&Bc)[NT] = (w % 2 == 0) ? B0 : B1;
      u32x4(&Bn)[NT] = (w % 2 == 0) ? B1 : B0;
      u32x4(&A)[MT] = (w % 2 == 0) ? A0 : A1;
      u32x4(&An)[MT] = (w % 2 == 0) ? A1 : A0;
      if (w + 1 < 4) {
        load_a(cur, An, w + 1);
        unpack(Bn, w + 1);
      }
      // keep the next word's reads ahead of this word's products (the
      // scheduler would otherwise sink each read to just before its use);
      // post-scaled, only for INT4 G = 128: with two groups per step, or the
      // NF4 table, the accumulators leave no registers for both buffers
      if constexpr (PATH == 0 || (FMT == 0 && GPT == 1)) __builtin_amdgcn_sched_barrier(0);
      products(A, Bc, w);
      if constexpr (PATH == 1) {
        if ((w % WPG) == WPG - 1) scale_group(w / WPG);
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
      const int m = m0 + mt * 16 + 4 * kb + i;
      if (m >= M) continue;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + wn * 32 + nt * 16 + ln;
        if (n >= N) continue;
        if (tpart)
          tpart[(((size_t)ks * gridDim.x + (place - tile0)) * kHBM + (m - m0)) * kHBN + (n - n0)] = C[mt][nt][i];
        else if (S == 1)
          y[(size_t)m * N + n] = float_to_half_bits(C[mt][nt][i]);
        else
          partial[((size_t)ks * M + m) * N + n] = C[mt][nt][i];
      }
    }
}

// S > 1: every tile split over S K slices into `partial` [S][M][N]; else the
// tail plan `tp` (tp.S > 1: the left-over tiles split into `tpart`).
template <int PATH, int FMT, int GPT>
int launch_f16(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
               const uint16_t* zero, uint16_t* y, float* partial, int S, const TailPlan& tp, float* tpart,
               hipStream_t s) {
  if ((size_t)M * K * 2 >= (1ull << 32))
    return fail(-2 /* W4_EUNSUPPORTED */, "w4_gemm: activations of %d x %d exceed the 4 GiB one call addresses", M, K);
  constexpr int kLds = kHStages * kHStage;
  const int st = allow_dynamic_lds(reinterpret_cast<const void*>(&gemm_f16_kernel<PATH, FMT, GPT>), kLds, "w4_gemm");
  if (st != 0) return st;
  const int tiles_m = (M + kHBM - 1) / kHBM, tiles_n = (N + kHBN - 1) / kHBN;
  const long tiles = (long)tiles_n * tiles_m;
  const int gm = gemm_group_rows();
  const bool tail = S == 1 && tp.S > 1 && tpart;
  const long main_tiles = tail ? tp.main : tiles;
  int st2;
  if (main_tiles > 0) {  // a tail-only plan has no full rounds
    hipLaunchKernelGGL((gemm_f16_kernel<PATH, FMT, GPT>), dim3((unsigned)main_tiles, (unsigned)S),
                       dim3(kF16Threads), kLds, s, x, M, K, N, packed, scale, zero, y, partial, nullptr, 0, gm);
    if ((st2 = check_launch("gemm")) != 0) return st2;
  }
  if (tail) {
    hipLaunchKernelGGL((gemm_f16_kernel<PATH, FMT, GPT>), dim3((unsigned)tp.r, (unsigned)tp.S), dim3(kF16Threads),
                       kLds, s, x, M, K, N, packed, scale, zero, y, nullptr, tpart, (int)tp.main, gm);
    if ((st2 = check_launch("gemm tail")) != 0) return st2;
    return launch_tail_reduce(tpart, tp, kHBM, kHBN, tiles_m, tiles_n, gm, M, N, y, s);
  }
  if (S == 1) return 0;
  return launch_reduce_partials(partial, S, (long)M * N, y, s);
}


// ---------------------------------------------------------------------------
// Multi-Scale Dequant path, on the fp16 kernel's frame: 128 tokens x 256
// weight rows per workgroup, the 8 waves side by side along N (each 128 x 32,
// so every widened weight operand serves 8 token tiles and both slices), and
// three stages of global -> LDS copies (both slices' tiles, the weight tiles
// and the scales).  The activation slices arrive from the decomposition kernel
// in the operand layout (per 64 K positions, lane kb's 16 bytes contiguous),
// so a token row of a step is 128 bytes = 8 chunks, stored at chunk
// c ^ (m % 8).  The zero point is folded into the weight operand exactly: per
// byte, ((q | 0x80) - z) ^ 0x80 is q - z in two's complement (no byte borrows,
// since 113 <= 128 + q - z <= 143), so each group's int32 product is
// D_j = sum A_j * (q - z) and the epilogue is C += s * (D_1 + r * D_2) with
// r = s_2 / s_1 per token; y = s_1 * C.
// With three slices, C += s * (D_1 + r_2 D_2 + r_3 D_3).  With the fixed
// ratio (two slices, s_2 = s_1 / 254) the products combine exactly in int32
// as E = 254 D_1 + D_2 (|E| < 2^26), one conversion per group: C += s * E,
// and the store multiplies by s_1 / 254.
// Token tiles per wave: 8 (128 tokens per workgroup) where the registers and
// the LDS allow, 4 for G = 64 with two slices, for three slices and for the
// test variant that also writes the integer products.
constexpr int msd_mt(int gpt, int ns, bool dbg) { return (!dbg && ns < 3 && (gpt == 1 || ns == 1)) ? 8 : 4; }

template <int GPT, int NS, bool DBG, bool FIXED>
__global__ __launch_bounds__(kF16Threads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_msd_kernel(
    const int8_t* __restrict__ slices, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    const float* __restrict__ tok_scale, int32_t* __restrict__ acc_out, float* __restrict__ tpart, int tile0,
    int gm) {
  constexpr int G = kStepK / GPT;
  constexpr int UPG = 2 / GPT;  // int8 products (64 K positions each) per group
  constexpr int MT = msd_mt(GPT, NS, DBG), NT = 2;
  constexpr int BM = 16 * MT;       // tokens per workgroup
  constexpr int kRowCopies = BM / 64;  // 8-row copies per wave per slice
  constexpr int kSlice = BM * 128;  // one slice's rows of a step
  constexpr int kA = NS * kSlice;
  constexpr int kStage = kA + kHB + kHS;
  static_assert(!FIXED || NS == 2, "the fixed ratio defines a second slice");
  constexpr int NR = (NS > 1 && !FIXED) ? NS - 1 : 1;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ float ratio[NR][BM];  // s_j / s_1 per tile row, j >= 2

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wn = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ln = lane % 16, kb = lane / 16;

  const int tiles_n = (N + kHBN - 1) / kHBN;
  const int place = tile0 + xcd_run(blockIdx.x, gridDim.x);
  int mb, nb;
  tile_mn(place, (M + BM - 1) / BM, tiles_n, gm, mb, nb);
  const int n0 = nb * kHBN;
  const int m0 = mb * BM;

  const int ng = K / G;
  const int KT = K / kStepK;
  const int ntile_last = N / 16 - 1;
  // K slice of this workgroup (gridDim.y > 1 only for a tail launch, whose
  // partials go to tpart)
  const int S = gridDim.y, ks = blockIdx.y;
  const int kt0 = (int)((long)KT * ks / S), kt1 = (int)((long)KT * (ks + 1) / S);

  if (tid < BM) {
    const int m = min(m0 + tid, M - 1);
    const float s1 = tok_scale[m];
#pragma unroll
    for (int j = 0; j < NR; ++j)
      ratio[j][tid] = (NS > 1 && !FIXED && s1 != 0.f) ? tok_scale[(size_t)(j + 1) * M + m] / s1 : 0.f;
  }

  // ---- copies.  Wave w fills rows [w BM/8, (w + 1) BM/8) of every slice (8
  // rows of 128 bytes per instruction), weight tiles 2 w and 2 w + 1, and its
  // share of the scale copies (as in the fp16 kernel).
  // slice j's descriptor, from a slice size kept in a scalar register (the
  // compiler otherwise may share the product with vector code and then has
  // to loop over lanes to form the descriptor)
  const uint32_t slice_bytes = __builtin_amdgcn_readfirstlane((uint32_t)M * (uint32_t)K);
  auto ar = [&](int j) { return make_rsrc(slices + (size_t)j * slice_bytes, slice_bytes); };
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(packed, (uint32_t)((size_t)N * (K / 2)));
  uint32_t voff_a[kRowCopies];
#pragma unroll
  for (int i = 0; i < kRowCopies; ++i) {
    const int row = wn * (BM / 8) + 8 * i + lane / 8;
    const int c = (lane % 8) ^ (row & 7);
    voff_a[i] = (uint32_t)(m0 + row) * (uint32_t)K + (uint32_t)c * 16;  // rows past M read zeros
  }
  uint32_t voff_b[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    voff_b[j] = (uint32_t)min(n0 / 16 + 2 * wn + j, ntile_last) * (uint32_t)KT * 1024 + (uint32_t)lane * 16;
  constexpr int kSCTotal = GPT * 2 * 4;
  constexpr int kSC = h_scale_copies(0, GPT);
  constexpr int kCopies = NS * kRowCopies + 2 + kSC;
  static_assert(kCopies < 16, "copy count must fit the low vmcnt field");
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scale, (uint32_t)((size_t)N * ng * 2));
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(zero, (uint32_t)((size_t)N * ng * 2));
  uint32_t voff_s[kSC];
  int sc_dst[kSC];
#pragma unroll
  for (int j = 0; j < kSC; ++j) {
    const int c = (wn * kSC + j) % kSCTotal;
    const int gi = c / 8, arr = (c / 4) % 2, quarter = c % 4;
    const int col = quarter * 64 + lane;
    voff_s[j] = (uint32_t)(n0 + col) * (uint32_t)ng * 2u + (uint32_t)gi * 2u;  // columns past N read zeros
    sc_dst[j] = kA + kHB + ((gi * 2 + arr) * kHBN + quarter * 64) * 4;
  }
  auto stage = [&](int kt) { return smem + ((kt - kt0) % kHStages) * kStage; };
  auto issue_step = [&](int kt) {
    unsigned char* st = stage(kt);
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < kRowCopies; ++i)
        copy16_to_lds(ar(j), voff_a[i], (uint32_t)kt * 128, st + j * kSlice + (wn * (BM / 8) + 8 * i) * 128);
#pragma unroll
    for (int j = 0; j < 2; ++j) copy16_to_lds(wr, voff_b[j], (uint32_t)kt * 1024, st + kA + (2 * wn + j) * 1024);
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      const int c = (wn * kSC + j) % kSCTotal;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(((c / 4) % 2) == 1 ? zr : sr, (lds_void*)(st + sc_dst[j]), 2,
                                               voff_s[j], (uint32_t)kt * GPT * 2u, 0, 0);
    }
  };
  auto wait_all_but_one_step = [&]() { __builtin_amdgcn_s_waitcnt(kCopies | (0x7 << 4) | (0xF << 8)); };

  f32x4 C[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) C[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

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

    const uint32_t* s_lds = reinterpret_cast<const uint32_t*>(cur + kA + kHB);
    u32x4 Bq[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Bq[nt] = *reinterpret_cast<const u32x4*>(cur + kA + (2 * wn + nt) * 1024 + lane * 16);

#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      u32x4 Bi[UPG][NT];
      float sv[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = wn * 32 + nt * 16 + ln;
        sv[nt] = half_bits_to_float((uint16_t)s_lds[(gi * 2) * kHBN + col]);
        const int zv = (int)half_bits_to_float((uint16_t)s_lds[(gi * 2 + 1) * kHBN + col]);
        const uint32_t zb = (uint32_t)zv * 0x01010101u;
#pragma unroll
        for (int u = 0; u < UPG; ++u) {
          const int pu = gi * UPG + u;
          const uint32_t w0 = Bq[nt][2 * pu], w1 = Bq[nt][2 * pu + 1];
          auto qz = [&](uint32_t q) { return ((q | 0x80808080u) - zb) ^ 0x80808080u; };  // bytes q - z
          Bi[u][nt] = u32x4{qz(w0 & 0x0F0F0F0Fu), qz((w0 >> 4) & 0x0F0F0F0Fu), qz(w1 & 0x0F0F0F0Fu),
                            qz((w1 >> 4) & 0x0F0F0F0Fu)};
        }
      }
      // slice fragments of token tile mt (both buffers: tile mt + 1's reads
      // are issued before tile mt's products)
      u32x4 Af[2][NS][UPG];
      auto load_frag = [&](u32x4 (&A)[NS][UPG], int mt) {
        const int row = mt * 16 + ln;
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
          for (int u = 0; u < UPG; ++u) {
            const int c = 4 * (gi * UPG + u) + kb;
            A[j][u] = *reinterpret_cast<const u32x4*>(cur + j * kSlice + row * 128 + ((c ^ (ln & 7)) << 4));
          }
      };
      load_frag(Af[0], 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt + 1 < MT) load_frag(Af[(mt + 1) % 2], mt + 1);
        __builtin_amdgcn_sched_barrier(0);
        i32x4 D[NS][NT];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            i32x4 d = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < UPG; ++u) d = mfma_i8(Af[mt % 2][j][u], Bi[u][nt], d);
            D[j][nt] = d;
          }
        }
        const int rloc = mt * 16 + 4 * kb;
        f32x4 rr[NR];
#pragma unroll
        for (int j = 0; j < NR; ++j) rr[j] = *reinterpret_cast<const f32x4*>(&ratio[j][rloc]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float e;
            if constexpr (FIXED) {
              e = (float)(__mul24(D[0][nt][i], 254) + D[1][nt][i]);
            } else {
              e = (float)D[0][nt][i];
#pragma unroll
              for (int j = 1; j < NS; ++j) e = fmaf(rr[j - 1][i], (float)D[j][nt][i], e);
            }
            C[mt][nt][i] = fmaf(sv[nt], e, C[mt][nt][i]);
          }
          if constexpr (DBG) {  // exact integer per-group products, zero point folded
            const int n = n0 + wn * 32 + nt * 16 + ln;
            const int g = kt * GPT + gi;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int m = m0 + rloc + i;
              if (m < M && n < N) {
#pragma unroll
                for (int j = 0; j < NS; ++j) acc_out[(((size_t)j * M + m) * ng + g) * N + n] = D[j][nt][i];
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
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
      const int m = m0 + mt * 16 + 4 * kb + i;
      if (m >= M) continue;
      const float s1 = tok_scale[FIXED ? (size_t)M + m : (size_t)m];  // s_1, or s_1 / 254
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + wn * 32 + nt * 16 + ln;
        if (n >= N) continue;
        if (tpart)
          tpart[(((size_t)ks * gridDim.x + (place - tile0)) * BM + (m - m0)) * kHBN + (n - n0)] = C[mt][nt][i] * s1;
        else
          y[(size_t)m * N + n] = float_to_half_bits(C[mt][nt][i] * s1);
      }
    }
}

template <int GPT, int NS, bool FIXED>
int launch_msd(const int8_t* slices, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
               const uint16_t* zero, uint16_t* y, const float* tok_scale, int32_t* acc_out, float* tpart,
               size_t tpart_bytes, hipStream_t s) {
  constexpr int kStage = NS * 16 * msd_mt(GPT, NS, false) * 128 + kHB + kHS;  // the larger of the two variants
  constexpr int kLds = kHStages * kStage;
  if ((size_t)NS * M * K >= (1ull << 32))
    return fail(-2 /* W4_EUNSUPPORTED */, "w4_gemm_decomp: slices of %d x %d exceed the 4 GiB one call addresses", M, K);
  const void* fn = acc_out ? reinterpret_cast<const void*>(&gemm_msd_kernel<GPT, NS, true, FIXED>)
                           : reinterpret_cast<const void*>(&gemm_msd_kernel<GPT, NS, false, FIXED>);
  const int st = allow_dynamic_lds(fn, kLds, "w4_gemm_decomp");
  if (st != 0) return st;
  const int bm = 16 * msd_mt(GPT, NS, acc_out != nullptr);
  const int tiles_m = (M + bm - 1) / bm, tiles_n = (N + kHBN - 1) / kHBN;
  const long tiles = (long)tiles_n * tiles_m;
  const int gm = gemm_group_rows();
  const TailPlan tp = plan_tail(tiles, K / kStepK, bm, kHBN);
  const bool tail = tp.S > 1 && tpart && tpart_bytes >= tp.bytes;
  const long main_tiles = tail ? tp.main : tiles;
  auto go = [&](dim3 grid, float* part, int tile0) {
    if (acc_out)
      hipLaunchKernelGGL((gemm_msd_kernel<GPT, NS, true, FIXED>), grid, dim3(kF16Threads), kLds, s, slices, M, K, N,
                         packed, scale, zero, y, tok_scale, acc_out, part, tile0, gm);
    else
      hipLaunchKernelGGL((gemm_msd_kernel<GPT, NS, false, FIXED>), grid, dim3(kF16Threads), kLds, s, slices, M, K, N,
                         packed, scale, zero, y, tok_scale, acc_out, part, tile0, gm);
  };
  int st2;
  if (main_tiles > 0) {
    go(dim3((unsigned)main_tiles), nullptr, 0);
    if ((st2 = check_launch("gemm_msd")) != 0) return st2;
  }
  if (!tail) return 0;
  go(dim3((unsigned)tp.r, (unsigned)tp.S), tpart, (int)tp.main);
  if ((st2 = check_launch("gemm_msd tail")) != 0) return st2;
  return launch_tail_reduce(tpart, tp, bm, kHBN, tiles_m, tiles_n, gm, M, N, y, s);
}

// ---------------------------------------------------------------------------
// Fixed-ratio Multi-Scale Dequant with the decomposition moved into the
// product's K loop.  A pre-pass computes only s_1 per token (the row absmax
// over 127); every K step copies the fp16 activation tile to LDS with the
// weight tiles and scales, and the workgroup turns it into the two int8 slices
// (the operand layout gemm_msd_kernel reads) before that step's products.  The
// slices never reach HBM; in exchange each workgroup column decides its rows
// again, N / 256 times per element.
//
// The decisions are taken in fp32 and equal the fp64 ones of the separate
// decomposition.  With inv = fp32(1 / s_1) (relative error <= 2^-24 plus the
// fp64 step's 2^-53), t_1 = fl32(x * inv) is within 127.0001 * 2^-23 <
// 2^-16 of x / s_1, and with r_1 = fl32(x - s_1 A_1) (one fused rounding) and
// t_2 = fl32(fl32(254 r_1) * inv), t_2 is within 127.0001 * 2^-22 < 2^-15
// of 254 r_1 / s_1 (|x| <= amax <= 127.00002 s_1, |r_1| <= s_1 / 2).  The fp64
// quotients are within 2^-46 of the exact ones.  So wherever t is at least
// 2^-14 away from every half-integer, rint(t) is the fp64 decision; elements
// closer than that (about 1 in 8000 per slice) are decided again exactly
// (exact_rint_f32).  rint and the byte come from one fp32 addition:
// for |t| < 2^22, fl32(t + 1.5 * 2^23) = 1.5 * 2^23 + rint(t) (ties to even),
// whose low byte is rint(t) in two's complement.
constexpr float kRintMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kNearHalf = 0x1p-14f;

// s_1 = fp32(max_k |x[m,k]| / 127) (the quotient in fp64) and its fixed-ratio
// partner fp32(s_1 / 254) per token row; one wave per row.
__global__ __launch_bounds__(256) void row_scale_kernel(const uint16_t* __restrict__ x, int M, int K,
                                                        float* __restrict__ tok_scale) {
  const int lane = threadIdx.x % kWave;
  const int m = blockIdx.x * 4 + threadIdx.x / kWave;
  if (m >= M) return;
  const uint16_t* xr = x + (size_t)m * K;
  float amax = 0.f;
  constexpr int kU = 4;
  for (int k0 = 8 * lane; k0 < K; k0 += kU * 8 * kWave) {
    u32x4 w[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int k = k0 + u * 8 * kWave;
      w[u] = k < K ? *reinterpret_cast<const u32x4*>(xr + k) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        amax = fmaxf(amax, fabsf(half_bits_to_float((uint16_t)(w[u][i] & 0xFFFFu))));
        amax = fmaxf(amax, fabsf(half_bits_to_float((uint16_t)(w[u][i] >> 16))));
      }
  }
  amax = wave_max(amax);
  if (lane == 0) {
    const double s1 = (double)(float)((double)amax / 127.0);
    tok_scale[m] = (float)s1;
    tok_scale[(size_t)M + m] = (float)(s1 / 254.0);
  }
}

// The two codes of one element (fp32 path; `near` is set when either quotient
// lies within kNearHalf of a half-integer).  Returns the bits of the clamped
// magic sums, whose low bytes are A_1 and A_2.
__device__ __forceinline__ void fixed_codes_f32(float xf, float s1, float inv, uint32_t& b1, uint32_t& b2,
                                                bool& near) {
#pragma clang fp contract(off)
  const float t1 = xf * inv;
  const float y1 = t1 + kRintMagic;
  const float e1 = t1 - (y1 - kRintMagic);
  near |= fabsf(fabsf(e1) - 0.5f) < kNearHalf;
  const float y1c = fminf(fmaxf(y1, kRintMagic - 127.f), kRintMagic + 127.f);
  const float r1 = fmaf(-s1, y1c - kRintMagic, xf);
  const float t2 = (254.f * r1) * inv;
  const float y2 = t2 + kRintMagic;
  const float e2 = t2 - (y2 - kRintMagic);
  near |= fabsf(fabsf(e2) - 0.5f) < kNearHalf;
  const float y2c = fminf(fmaxf(y2, kRintMagic - 127.f), kRintMagic + 127.f);
  b1 = __float_as_uint(y1c);
  b2 = __float_as_uint(y2c);
}

// rint((v - c s_1) / s_1) decided exactly from an estimate t within 1/4 of
// the quotient: the half-integer next to rint(t) on t's side is the only
// boundary that can lie between them, and the sign of v - (c + boundary) s_1,
// computed exactly and rounded once, tells on which side the quotient lies
// (on the boundary: to even).  v and c + boundary are exact in fp32 here.
// The fp64 decomposition decides rint(fl64(quotient)); the two agree because
// no quotient here lies within 2^-25 of a half-integer without being one (its
// distance is a multiple of the finer of the grids of x and s_1 / 2, divided
// by s_1), while fl64 moves it by at most 2^-46.
__device__ __forceinline__ float exact_rint_f32(float v, float c, float s1, float t) {
#pragma clang fp contract(off)
  const float q = (t + kRintMagic) - kRintMagic;
  const float sg = t >= q ? 1.f : -1.f;
  const float hb = q + 0.5f * sg;
  const float d = fmaf(-(c + hb), s1, v);
  const bool odd = ((int)q & 1) != 0;
  return (d * sg > 0.f || (d == 0.f && odd)) ? q + sg : q;
}

template <int GPT>
__global__ __launch_bounds__(kF16Threads) __attribute__((amdgpu_waves_per_eu(2, 2))) void gemm_msd_fused_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    const float* __restrict__ tok_scale, float* __restrict__ tpart, int tile0, int gm) {
  constexpr int G = kStepK / GPT;
  constexpr int UPG = 2 / GPT;
  constexpr int MT = msd_mt(GPT, 2, false), NT = 2;
  constexpr int BM = 16 * MT;
  constexpr int kX = BM * 256;             // fp16 activation tile of a step
  constexpr int kXCopies = BM / 32;        // 4 rows of 256 bytes per copy, BM / 8 rows per wave
  constexpr int kSlice = BM * 128;         // one slice's rows of a step
  constexpr int kStage = kX + kHB + kHS;   // two stages, then the two slices
  constexpr int kTPR = kF16Threads / BM;   // threads per row in the conversion
  constexpr int kCPT = 8 / kTPR;           // 16-byte operand chunks per thread per slice
  extern __shared__ __align__(16) unsigned char smem[];
  unsigned char* const slices = smem + 2 * kStage;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wn = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int ln = lane % 16, kb = lane / 16;

  const int tiles_n = (N + kHBN - 1) / kHBN;
  const int place = tile0 + xcd_run(blockIdx.x, gridDim.x);
  int mb, nb;
  tile_mn(place, (M + BM - 1) / BM, tiles_n, gm, mb, nb);
  const int n0 = nb * kHBN;
  const int m0 = mb * BM;
  const int ng = K / G;
  const int KT = K / kStepK;
  const int ntile_last = N / 16 - 1;
  const int S = gridDim.y, ks = blockIdx.y;
  const int kt0 = (int)((long)KT * ks / S), kt1 = (int)((long)KT * (ks + 1) / S);

  // this thread's conversion row and its scale (rows past M: zeros)
  const int crow = tid / kTPR, cq = tid % kTPR;
  const float s1r = m0 + crow < M ? tok_scale[m0 + crow] : 0.f;
  const float invr = s1r != 0.f ? (float)(1.0 / (double)s1r) : 0.f;

  // ---- copies: wave w fills activation rows [w BM/8, (w + 1) BM/8) (4 rows
  // of 256 bytes per copy; row r's 16-byte chunk c lands at slot
  // c ^ 4 (r mod 4), which keeps the conversion's reads free of bank
  // conflicts), weight tiles 2 w and 2 w + 1, and its share of the scales.
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(packed, (uint32_t)((size_t)N * (K / 2)));
  uint32_t voff_x[kXCopies];
#pragma unroll
  for (int i = 0; i < kXCopies; ++i) {
    const int row = wn * (BM / 8) + 4 * i + lane / 16;
    const int c = (lane % 16) ^ ((row & 3) << 2);
    voff_x[i] = (uint32_t)(m0 + row) * (uint32_t)K * 2u + (uint32_t)c * 16u;  // rows past M read zeros
  }
  uint32_t voff_b[2];
#pragma unroll
  for (int j = 0; j < 2; ++j)
    voff_b[j] = (uint32_t)min(n0 / 16 + 2 * wn + j, ntile_last) * (uint32_t)KT * 1024 + (uint32_t)lane * 16;
  constexpr int kSCTotal = GPT * 2 * 4;
  constexpr int kSC = h_scale_copies(0, GPT);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(scale, (uint32_t)((size_t)N * ng * 2));
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(zero, (uint32_t)((size_t)N * ng * 2));
  uint32_t voff_s[kSC];
  int sc_dst[kSC];
#pragma unroll
  for (int j = 0; j < kSC; ++j) {
    const int c = (wn * kSC + j) % kSCTotal;
    const int gi = c / 8, quarter = c % 4;
    const int col = quarter * 64 + lane;
    voff_s[j] = (uint32_t)(n0 + col) * (uint32_t)ng * 2u + (uint32_t)gi * 2u;
    sc_dst[j] = kX + kHB + ((gi * 2 + (c / 4) % 2) * kHBN + quarter * 64) * 4;
  }
  auto stage = [&](int kt) { return smem + ((kt - kt0) % 2) * kStage; };
  auto issue_step = [&](int kt) {
    unsigned char* st = stage(kt);
#pragma unroll
    for (int i = 0; i < kXCopies; ++i)
      copy16_to_lds(xr, voff_x[i], (uint32_t)kt * 256, st + (wn * (BM / 8) + 4 * i) * 256);
#pragma unroll
    for (int j = 0; j < 2; ++j) copy16_to_lds(wr, voff_b[j], (uint32_t)kt * 1024, st + kX + (2 * wn + j) * 1024);
#pragma unroll
    for (int j = 0; j < kSC; ++j) {
      const int c = (wn * kSC + j) % kSCTotal;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(((c / 4) % 2) == 1 ? zr : sr, (lds_void*)(st + sc_dst[j]), 2,
                                               voff_s[j], (uint32_t)kt * GPT * 2u, 0, 0);
    }
  };
  // the step's activation tile -> both slices in operand order: thread
  // (row, q) writes operand chunks c = q + kTPR i of its row (K positions
  // 64 b + 8 kb + 0..7 and 64 b + 32 + 8 kb + 0..7, c = 4 b + kb)
  auto convert = [&](const unsigned char* xs) {
#pragma unroll
    for (int i = 0; i < kCPT; ++i) {
      const int c = cq + kTPR * i;
      const int b = c / 4, kq = c % 4;
      uint32_t d1[4], d2[4];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int xc = 8 * b + 4 * h + kq;
        const u32x4 w = *reinterpret_cast<const u32x4*>(xs + crow * 256 + ((xc ^ ((crow & 3) << 2)) << 4));
        uint32_t b1[8], b2[8];
        bool near = false;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          fixed_codes_f32(half_bits_to_float((uint16_t)(w[e / 2] >> (16 * (e % 2)))), s1r, invr, b1[e], b2[e],
                          near);
        if (near) {  // rare: decide this piece's codes exactly
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float xf = half_bits_to_float((uint16_t)(w[e / 2] >> (16 * (e % 2))));
            const float a1 = fminf(fmaxf(exact_rint_f32(xf, 0.f, s1r, xf * invr), -127.f), 127.f);
            const float r1 = fmaf(-s1r, a1, xf);
            const float a2 =
                fminf(fmaxf(exact_rint_f32(254.f * xf, 254.f * a1, s1r, (254.f * r1) * invr), -127.f), 127.f);
            b1[e] = (uint32_t)(int)a1;
            b2[e] = (uint32_t)(int)a2;
          }
        }
        // operand byte order e0 e4 e1 e5 | e2 e6 e3 e7 (low bytes of the codes)
        auto pack = [](uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3) {
          return perm_b32(perm_b32(p3, p2, 0x0c0c0400u), perm_b32(p1, p0, 0x0c0c0400u), 0x05040100u);
        };
        d1[2 * h] = pack(b1[0], b1[4], b1[1], b1[5]);
        d1[2 * h + 1] = pack(b1[2], b1[6], b1[3], b1[7]);
        d2[2 * h] = pack(b2[0], b2[4], b2[1], b2[5]);
        d2[2 * h + 1] = pack(b2[2], b2[6], b2[3], b2[7]);
      }
      const int off = crow * 128 + ((c ^ (crow & 7)) << 4);
      *reinterpret_cast<u32x4*>(slices + off) = u32x4{d1[0], d1[1], d1[2], d1[3]};
      *reinterpret_cast<u32x4*>(slices + kSlice + off) = u32x4{d2[0], d2[1], d2[2], d2[3]};
    }
  };

  f32x4 C[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) C[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  issue_step(kt0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int kt = kt0; kt < kt1; ++kt) {
    const unsigned char* cur = stage(kt);
    if (kt + 1 < kt1) issue_step(kt + 1);  // into the stage step kt - 1 used, read by everyone before the barrier
    convert(cur);
    lds_barrier();  // the slices are written

    const uint32_t* s_lds = reinterpret_cast<const uint32_t*>(cur + kX + kHB);
    u32x4 Bq[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) Bq[nt] = *reinterpret_cast<const u32x4*>(cur + kX + (2 * wn + nt) * 1024 + lane * 16);
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      u32x4 Bi[UPG][NT];
      float sv[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int col = wn * 32 + nt * 16 + ln;
        sv[nt] = half_bits_to_float((uint16_t)s_lds[(gi * 2) * kHBN + col]);
        const int zv = (int)half_bits_to_float((uint16_t)s_lds[(gi * 2 + 1) * kHBN + col]);
        const uint32_t zb = (uint32_t)zv * 0x01010101u;
#pragma unroll
        for (int u = 0; u < UPG; ++u) {
          const int pu = gi * UPG + u;
          const uint32_t w0 = Bq[nt][2 * pu], w1 = Bq[nt][2 * pu + 1];
          auto qz = [&](uint32_t q) { return ((q | 0x80808080u) - zb) ^ 0x80808080u; };
          Bi[u][nt] = u32x4{qz(w0 & 0x0F0F0F0Fu), qz((w0 >> 4) & 0x0F0F0F0Fu), qz(w1 & 0x0F0F0F0Fu),
                            qz((w1 >> 4) & 0x0F0F0F0Fu)};
        }
      }
      u32x4 Af[2][2][UPG];
      auto load_frag = [&](u32x4 (&A)[2][UPG], int mt) {
        const int row = mt * 16 + ln;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int u = 0; u < UPG; ++u) {
            const int c = 4 * (gi * UPG + u) + kb;
            A[j][u] = *reinterpret_cast<const u32x4*>(slices + j * kSlice + row * 128 + ((c ^ (ln & 7)) << 4));
          }
      };
      load_frag(Af[0], 0);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        if (mt + 1 < MT) load_frag(Af[(mt + 1) % 2], mt + 1);
        __builtin_amdgcn_sched_barrier(0);
        i32x4 D[2][NT];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            i32x4 d = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int u = 0; u < UPG; ++u) d = mfma_i8(Af[mt % 2][j][u], Bi[u][nt], d);
            D[j][nt] = d;
          }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            C[mt][nt][i] = fmaf(sv[nt], (float)(__mul24(D[0][nt][i], 254) + D[1][nt][i]), C[mt][nt][i]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of step kt + 1 have landed
    lds_barrier();                  // everyone's have; the slices and this stage are free again
  }

#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + mt * 16 + 4 * kb + i;
      if (m >= M) continue;
      const float s1 = tok_scale[(size_t)M + m];  // s_1 / 254
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int n = n0 + wn * 32 + nt * 16 + ln;
        if (n >= N) continue;
        if (tpart)
          tpart[(((size_t)ks * gridDim.x + (place - tile0)) * BM + (m - m0)) * kHBN + (n - n0)] = C[mt][nt][i] * s1;
        else
          y[(size_t)m * N + n] = float_to_half_bits(C[mt][nt][i] * s1);
      }
    }
}

template <int GPT>
int launch_msd_fused(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                     const uint16_t* zero, uint16_t* y, const float* tok_scale, float* tpart, size_t tpart_bytes,
                     hipStream_t s) {
  constexpr int BM = 16 * msd_mt(GPT, 2, false);
  constexpr int kLds = 2 * (BM * 256 + kHB + kHS) + 2 * BM * 128;
  const void* fn = reinterpret_cast<const void*>(&gemm_msd_fused_kernel<GPT>);
  const int st = allow_dynamic_lds(fn, kLds, "w4_gemm_decomp_fixed_fused");
  if (st != 0) return st;
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + kHBN - 1) / kHBN;
  const long tiles = (long)tiles_n * tiles_m;
  const int gm = gemm_group_rows();
  const TailPlan tp = plan_tail(tiles, K / kStepK, BM, kHBN);
  const bool tail = tp.S > 1 && tpart && tpart_bytes >= tp.bytes;
  const long main_tiles = tail ? tp.main : tiles;
  int st2;
  if (main_tiles > 0) {
    hipLaunchKernelGGL((gemm_msd_fused_kernel<GPT>), dim3((unsigned)main_tiles), dim3(kF16Threads), kLds, s, x, M, K,
                       N, packed, scale, zero, y, tok_scale, nullptr, 0, gm);
    if ((st2 = check_launch("gemm_msd_fused")) != 0) return st2;
  }
  if (!tail) return 0;
  hipLaunchKernelGGL((gemm_msd_fused_kernel<GPT>), dim3((unsigned)tp.r, (unsigned)tp.S), dim3(kF16Threads), kLds, s,
                     x, M, K, N, packed, scale, zero, y, tok_scale, tpart, (int)tp.main, gm);
  if ((st2 = check_launch("gemm_msd_fused tail")) != 0) return st2;
  return launch_tail_reduce(tpart, tp, BM, kHBN, tiles_m, tiles_n, gm, M, N, y, s);
}

}  // namespace

// K slices for the fp16 GEMM: while the grid holds fewer than about 192
// workgroups (256 CUs), double S as long as every slice keeps at least 4
// steps.  M = 256 layers: N = 8192 has 64 tiles -> S = 4.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 0;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) {
      (void)hipGetLastError();
      v = -1;
    }
    cache[dev].store(v, std::memory_order_relaxed);
  }
  return v > 0 ? v : 0;
}

TailPlan plan_tail(long tiles, int KT, int bm, int bn) {
  TailPlan p{tiles, 0, 1, 0};
  const char* e = std::getenv("W4_GEMM_TAIL");
  if (e && *e == '0') return p;
  const int C = device_cus();
  if (C <= 0 || tiles < 1) return p;
  const int r = (int)(tiles % C == 0 ? 0 : tiles % C);
  if (r == 0) return p;
  int S = 1;
  while ((long)r * S * 2 <= C && KT / (S * 2) >= 4) S *= 2;
  if (S == 1) return p;
  p.main = tiles - r;
  p.r = r;
  p.S = S;
  p.bytes = (size_t)S * r * bm * bn * sizeof(float);
  return p;
}

namespace {
// y at the tail tiles' outputs = fp16 of the sum over the S slices' partials,
// in slice order; thread i takes element i of the tail's [r][bm][bn].
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float* __restrict__ tpart, int S, int r, int tile0,
                                                          int bm, int bn, int tiles_m, int tiles_n, int gm, int M,
                                                          int N, uint16_t* __restrict__ y) {
  const long per = (long)bm * bn;
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (i >= (long)r * per) return;
  const int t = (int)(i / per);
  const int e = (int)(i - (long)t * per);
  int mb, nb;
  tile_mn(tile0 + t, tiles_m, tiles_n, gm, mb, nb);
  const int m = mb * bm + e / bn, n = nb * bn + e % bn;
  if (m >= M || n >= N) return;
  float acc = 0.f;
  for (int k = 0; k < S; ++k) acc += tpart[(size_t)k * r * per + i];
  y[(size_t)m * N + n] = float_to_half_bits(acc);
}
}  // namespace

int launch_tail_reduce(const float* tpart, const TailPlan& tp, int bm, int bn, int tiles_m, int tiles_n, int gm,
                       int M, int N, uint16_t* y, hipStream_t s) {
  const long n = (long)tp.r * bm * bn;
  hipLaunchKernelGGL(tail_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tpart, tp.S, tp.r,
                     (int)tp.main, bm, bn, tiles_m, tiles_n, gm, M, N, y);
  return check_launch("gemm tail reduce");
}

int gemm_split(int M, int K, int N) {
  const int KT = K / kStepK;
  const long tiles = (long)((N + kHBN - 1) / kHBN) * ((M + kHBM - 1) / kHBM);
  int S = 1;
  const char* e = std::getenv("W4_GEMM_S");
  if (e && *e && std::atoi(e) >= 1) return std::min(std::atoi(e), KT);
  while (tiles * S < 192 && KT / (2 * S) >= 4) S *= 2;
  return S;
}

size_t gemm_workspace_bytes(int M, int K, int N) {
  const int S = gemm_split(M, K, N);
  if (S > 1) return (size_t)S * M * N * sizeof(float);
  const long tiles = (long)((N + kHBN - 1) / kHBN) * ((M + kHBM - 1) / kHBM);
  return plan_tail(tiles, K / kStepK, kHBM, kHBN).bytes;
}

int launch_gemm(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                const uint16_t* zero, int G, int fmt, int mode, uint16_t* y, void* ws, size_t ws_bytes,
                hipStream_t s) {
  int S = gemm_split(M, K, N);
  if (S > 1 && (!ws || ws_bytes < (size_t)S * M * N * sizeof(float))) S = 1;  // no room for partials: unsplit
  float* partial = S > 1 ? static_cast<float*>(ws) : nullptr;
  const long tiles = (long)((N + kHBN - 1) / kHBN) * ((M + kHBM - 1) / kHBM);
  TailPlan tp = plan_tail(tiles, K / kStepK, kHBM, kHBN);
  if (S > 1 || !ws || ws_bytes < tp.bytes) tp = TailPlan{tiles, 0, 1, 0};  // no room for the tail: one launch
  float* tpart = tp.S > 1 ? static_cast<float*>(ws) : nullptr;
#define W4_GEMM_CASE(PATH, FMT, GPT) \
  return launch_f16<PATH, FMT, GPT>(x, M, K, N, packed, scale, zero, y, partial, S, tp, tpart, s)
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
  (void)G;
  const size_t slices = ((size_t)nslices * M * K + 255) / 256 * 256;  // operand layout
  const size_t scales = ((size_t)nslices * M * sizeof(float) + 255) / 256 * 256;
  return slices + scales;
}

size_t decomp_tail_bytes(int M, int K, int N, int G, int nslices) {
  const int bm = 16 * msd_mt(G == 64 ? 2 : 1, nslices, false);
  const long tiles = (long)((N + kHBN - 1) / kHBN) * ((M + bm - 1) / bm);
  return plan_tail(tiles, K / kStepK, bm, kHBN).bytes;
}

int launch_gemm_decomp(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                       const uint16_t* zero, int G, int nslices, bool fixed, uint16_t* y, int8_t* slices_op,
                       int8_t* slices_out, float* tok_scale, int32_t* acc_out, float* tpart, size_t tpart_bytes,
                       hipStream_t s) {
  int st = launch_decompose(x, M, K, nslices, fixed, slices_op, slices_out, tok_scale, s);
  if (st != 0) return st;
#define W4_MSD(NS, FX)                                                                                             \
  return G == 64 ? launch_msd<2, NS, FX>(slices_op, M, K, N, packed, scale, zero, y, tok_scale, acc_out, tpart,   \
                                         tpart_bytes, s)                                                          \
                 : launch_msd<1, NS, FX>(slices_op, M, K, N, packed, scale, zero, y, tok_scale, acc_out, tpart,   \
                                         tpart_bytes, s)
  if (fixed) W4_MSD(2, true);
  if (nslices == 1) W4_MSD(1, false);
  if (nslices == 2) W4_MSD(2, false);
  W4_MSD(3, false);
#undef W4_MSD
}

size_t decomp_fused_workspace_bytes(int M) { return ((size_t)2 * M * sizeof(float) + 255) / 256 * 256; }

int launch_gemm_decomp_fused(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                             const uint16_t* zero, int G, uint16_t* y, float* tok_scale, float* tpart,
                             size_t tpart_bytes, hipStream_t s) {
  if ((size_t)M * K * 2 >= (1ull << 32))
    return fail(-2 /* W4_EUNSUPPORTED */, "w4_gemm_decomp_fixed_fused: x of %d x %d exceeds the 4 GiB one call addresses",
                M, K);
  hipLaunchKernelGGL(row_scale_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, x, M, K, tok_scale);
  int st = check_launch("row_scale");
  if (st != 0) return st;
  return G == 64 ? launch_msd_fused<2>(x, M, K, N, packed, scale, zero, y, tok_scale, tpart, tpart_bytes, s)
                 : launch_msd_fused<1>(x, M, K, N, packed, scale, zero, y, tok_scale, tpart, tpart_bytes, s);
}

}  // namespace w4

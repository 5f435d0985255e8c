// Decode-shaped W4 product y[M][N] = x[M][K] . W' for 1 <= M <= 32.
//
// The weight stream dominates: every packed byte is read once from HBM and
// turned into matrix-core operands on chip.  Dequantization follows the
// per-group product ("MixPE: Quantization and Hardware Co-design for Efficient
// LLM Inference", Abstract): each group's partial product is formed from the
// raw codes and multiplied by the group scale once.  NF4 levels come from a
// small table in LDS, as the "Fast NF4 Dequantization Kernels for Large
// Language Model Inference" page (Abstract) keeps its codebook in shared
// memory; here the table is indexed by a whole byte, so one lookup yields the
// pair of fp16 levels of two adjacent weights.
//
// Weight stream.  The packed weights are stored as tiles of 16 rows x 128
// K positions, 1024 contiguous bytes each, in which lane l of a wave finds
// its matrix-core B operands for the tile in bytes 16 l .. 16 l + 15 (word t:
// 8 codes of row l % 16 at K positions 32 t + 8 (l / 16) + 0..7).  A wave
// therefore streams a tile with one 16-byte load per lane and needs no
// on-chip transpose; tiles are prefetched R deep into a register ring.
//
// Work split.  Grid = (row blocks of 16*NWR weight rows) x (S slices of K).  A
// workgroup has NWR x NWK waves: wave (wr, wk) owns one 16-row tile column
// and a contiguous run of the slice's tiles.  The workgroup first stages in
// LDS, once, everything its waves share: the activation slice, already laid
// out as matrix-core A operands, and the rows' scales and zero points.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_f16): weight rows are the MFMA "n"
// dimension, tokens the "m" dimension.  Word t of a lane's 16 bytes feeds one
// product over K positions 32 t .. 32 t + 31 of the tile.  Token rows past M
// read row M-1 (never stored), which keeps every load unconditional.
//
// INT4 operands.  A code q in the low nibble of an fp16 lane is the subnormal
// value q * 2^-24 exactly, and in bits 4..7 it is q * 2^-20; masking the packed
// word therefore yields exact fp16 operands in 5 VALU ops per 8 codes, with no
// offset to cancel.  With the stored nibble order the masks yield the pairs
// (c0, c1), (c2, c3) * 16, (c4, c5), (c6, c7) * 16; the activations of the
// scaled pairs are staged pre-scaled by 1/16, so every product is
// x*q*2^-24.  The zero point is applied with the group's activation sum:
// y += s * (2^24 * sum x*q - z * sum x).
//
// Split K.  With S > 1 each workgroup stores its fp32 partial in the workspace
// with plain stores, and a small second kernel on the same stream adds the S
// partials in slice order and writes y.  Results are deterministic, the
// workspace needs no initial contents, and no workgroup waits on another (a
// last-arrival protocol through device-scope atomics costs several
// microseconds of serial latency at the end of every launch).
#include "w4_device.h"
#include "w4_internal.h"

#include <cstdlib>

namespace w4 {
namespace {

constexpr int kGemvMaxThreads = 512;
constexpr int kRing = 4;       // weight tiles in flight per wave (default depth of the staged kernel's ring)
constexpr int kXUMax = 8;      // staged activation units (16 B) per thread, at most
constexpr int kXUSmall = 4;    // the smaller staging batch (fewer redundant loads)
constexpr int kSE = 8;         // scale entries per lane, at most: 16 rows x 32 tiles per wave
constexpr int kMaxRun = kSE * kWave / 16;  // tiles per wave, at most
constexpr int kLutCopies = 16;  // copies of the NF4 pair table (16 KB of LDS)
// With one workgroup per CU and LDS to spare, 64 copies (64 KB): entry e of
// copy c at byte 256 e + 4 c, lane l reads copy l, so no lookup shares a
// bank and one v_perm_b32 forms a lookup's whole address (the code byte over
// the lane's copy offset).
constexpr int kLutCopiesWide = 64;

// NF4 level pair of code byte I (0..3) of word a from a table of LC copies
// (LC = 16: lut_c = lut + lane % 16; LC = 64: lane4 = 4 lane, the byte
// offset of the lane's copy)
template <int LC, int I>
__device__ __forceinline__ uint32_t lut_pair(const uint32_t* lut, const uint32_t* lut_c, uint32_t lane4, uint32_t a) {
  if constexpr (LC == kLutCopiesWide) {
    return *reinterpret_cast<const uint32_t*>(reinterpret_cast<const char*>(lut) +
                                              __builtin_amdgcn_perm(a, lane4, 0x0C0C0400u + 0x100u * I));
  } else {
    return lut_c[((a >> (8 * I)) & 0xFFu) * LC];
  }
}
constexpr int kSEDirect = 8;    // scale entries per lane in the direct variant
constexpr int kDirectFromM = 4; // the direct variant serves M > 4
constexpr int kTileK = 128;      // K positions per weight tile
constexpr int kTileBytes = 1024;  // 16 rows x 128 codes

// fp16 pair constants
constexpr uint32_t kHalfSixteenthPair = 0x2C002C00u;  // (1/16, 1/16)

__device__ __forceinline__ uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, a) * __builtin_bit_cast(h2, b));
}
__device__ __forceinline__ float lo_half(uint32_t w) { return half_bits_to_float((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float hi_half(uint32_t w) { return half_bits_to_float((uint16_t)(w >> 16)); }

// Interleave the low (sel 0x05040100) or high (0x07060302) fp16 halves of two
// activation words: result = half(a) | half(b) << 16.
__device__ __forceinline__ uint32_t pair_lo(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pair_hi(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

// u / d and u % d for 0 <= u < 2^22, 0 < d < 2^16, from a float reciprocal and
// one correction step (the float estimate is off by at most one).
__device__ __forceinline__ void div_small(int u, int d, float inv_d, int& q, int& r) {
  q = (int)((float)u * inv_d);
  r = u - q * d;
  if (r < 0) {
    --q;
    r += d;
  } else if (r >= d) {
    ++q;
    r -= d;
  }
}

// Cross-wave reduction over the NWK waves of a workgroup (through `red`, NWR x
// NWK x MT x 256 floats of LDS, free when called after a barrier), then the
// fp16 store, or with S > 1 the fp32 partial of this K slice (summed over the
// slices by gemv_reduce_kernel, launched right after on the same stream).
template <int MT, int TM = 0>
__device__ __forceinline__ void gemv_finish(const f32x4 (&C)[MT], float* red, int wave, int lane, int nwr, int nwk,
                                            int row_wg0, int M, int N, uint16_t* __restrict__ y,
                                            float* __restrict__ partial) {
  constexpr int kTile = MT * 256;
  const int S = gridDim.y;
  const int ks = blockIdx.y;
  if constexpr (TM == 2) {
    // 2 <= M <= 4: token j sits in product row 4 j, so lane l holds token
    // l / 16 of column l % 16 in its first accumulator element
    red[wave * 64 + lane] = C[0][0];
    __syncthreads();
    for (int e = threadIdx.x; e < 64 * nwr; e += blockDim.x) {
      const int w_r = e / 64, l = e % 64;
      const int m = l / 16, n = row_wg0 + 16 * w_r + l % 16;
      if (m >= M || n >= N) continue;
      float sum = 0.f;
      for (int k2 = 0; k2 < nwk; ++k2) sum += red[(k2 * nwr + w_r) * 64 + l];
      if (S == 1)
        y[(size_t)m * N + n] = float_to_half_bits(sum);
      else
        partial[((size_t)ks * M + m) * N + n] = sum;
    }
    return;
  }
  if constexpr (TM == 1) {
    // M = 1: only token 0 is live, in lanes 0..15 (row l) of each wave
    if (lane < 16) red[wave * 16 + lane] = C[0][0];
    __syncthreads();
    const int e = threadIdx.x;
    if (e < 16 * nwr) {
      const int w_r = e / 16, n = row_wg0 + e;
      if (n < N) {
        float sum = 0.f;
        for (int k2 = 0; k2 < nwk; ++k2) sum += red[(k2 * nwr + w_r) * 16 + e % 16];
        if (S == 1)
          y[n] = float_to_half_bits(sum);
        else
          partial[(size_t)ks * N + n] = sum;
      }
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave * kTile + (t * 4 + i) * 64 + lane] = C[t][i];
  __syncthreads();

  // element e of the workgroup's output (nwr tiles of 16 rows x 16*MT tokens)
  const int total = nwr * kTile;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int w_r = e / kTile;
    const int el = e - w_r * kTile;
    const int l = el % 64;
    const int i = (el / 64) % 4;
    const int t = el / 256;
    const int n = row_wg0 + 16 * w_r + l % 16;
    const int m = t * 16 + 4 * (l / 16) + i;
    if (m >= M || n >= N) continue;
    float sum = 0.f;
    for (int k2 = 0; k2 < nwk; ++k2) sum += red[(k2 * nwr + w_r) * kTile + el];
    if (S == 1)
      y[(size_t)m * N + n] = float_to_half_bits(sum);
    else
      partial[((size_t)ks * M + m) * N + n] = sum;
  }
}

// y = the sum of the S fp32 partials, in slice order (deterministic), rounded
// to fp16; 4 outputs per thread.
__global__ __launch_bounds__(256) void gemv_reduce_kernel(const float* __restrict__ partial, int S, long MN,
                                                          uint16_t* __restrict__ y) {
  const long i = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i >= MN) return;
  if (i + 4 <= MN) {
    f32x4 acc = *reinterpret_cast<const f32x4*>(partial + i);
    for (int k = 1; k < S; ++k) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(partial + (size_t)k * MN + i);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += v[j];
    }
    const uint32_t lo = (uint32_t)float_to_half_bits(acc[0]) | ((uint32_t)float_to_half_bits(acc[1]) << 16);
    const uint32_t hi = (uint32_t)float_to_half_bits(acc[2]) | ((uint32_t)float_to_half_bits(acc[3]) << 16);
    *reinterpret_cast<uint2*>(y + i) = uint2{lo, hi};
  } else {
    for (long e = i; e < MN; ++e) {
      float acc = partial[e];
      for (int k = 1; k < S; ++k) acc += partial[(size_t)k * MN + e];
      y[e] = float_to_half_bits(acc);
    }
  }
}

// Staged kernel.  TM (token mode), with one token tile: 1 for M == 1 (only
// the accumulator of token 0 is updated); 2 for 2 <= M <= 4, where token j
// is placed in product row 4 j (rows 4 j + 1 .. 4 j + 3 repeat it), so each
// lane's first accumulator element holds one token and the per-tile
// epilogue updates one element, not four.
// VS: the workgroup stages its rows' scale block for all of K with 16-byte
// loads (K not split, K / G a multiple of 8); otherwise each wave stages the
// block of its own run.
template <int FMT, int LB, int MT, int XU, int R, int TM, bool VS, int LC>
__global__ __launch_bounds__(kGemvMaxThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    float* __restrict__ partial, int nwr, int nwk, int sc_pitch, int x_bytes) {
  constexpr int G = 8 * LB;
  constexpr int GPT = kTileK / G;  // groups per tile: 1 (G=128) or 2 (G=64)
  constexpr int WPG = 4 / GPT;     // 4-byte words (one product each) per group
  constexpr int RG = G / 8;        // 8-position activation units per group
  static_assert(TM == 0 || MT == 1, "M <= 4 has one token tile");
  constexpr bool ONE = TM == 1;
  extern __shared__ __align__(16) unsigned char smem[];
  // NF4 pair table, kLutCopies interleaved copies: entry e of copy c at word
  // e * kLutCopies + c, and lane l reads copy l % kLutCopies, so random
  // indices from the lanes of a copy group spread over the banks instead of
  // colliding (one copy costs several conflict cycles per lookup).
  __shared__ uint32_t lut[FMT == 1 ? 256 * LC : 1];

  const int lane = threadIdx.x % kWave;
  // wave-uniform by construction; readfirstlane lets the compiler keep it (and
  // everything derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wr = wave % nwr;
  const int wk = wave / nwr;
  const int ln = lane % 16;
  const int kb = lane / 16;
  const int ng = K / G;
  const int KT = K / kTileK;  // tiles per 16-row tile column
  const int rows_wg = 16 * nwr;
  const int row_wg0 = blockIdx.x * rows_wg;
  const int S = gridDim.y;
  const int ks = blockIdx.y;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;

  // tile ranges: the workgroup's slice [ts0, ts1), the wave's run [t0, t0 + cnt)
  const int ts0 = (int)((long)KT * ks / S), ts1 = (int)((long)KT * (ks + 1) / S);
  const int t0 = ts0 + (int)((long)(ts1 - ts0) * wk / nwk);
  const int cnt = ts0 + (int)((long)(ts1 - ts0) * (wk + 1) / nwk) - t0;
  const int t_last = t0 + max(cnt, 1) - 1;
  const int k0 = ts0 * kTileK;  // first K position of the slice
  // this wave's tile column; a wave past the last one (only in a partial last
  // row block) re-reads the last column and stores nothing
  const int colw = min(row_wg0 / 16 + wr, N / 16 - 1);

  // Staging.  The whole slice's activations are staged once, as units of 8
  // consecutive K positions of one token: unit u = r M + m is chunk r of the
  // slice (K positions k0 + 8 r .. + 7) of token m, and u is also its 16-byte
  // slot (consecutive threads store consecutive slots).  Unit r = 16 tl + kb +
  // 4 w of tile tl is the A operand of lane (kb, m) for word w.  The plan keeps
  // the slice within XU units per thread, so it is loaded in one batch of
  // straight-line code whose waits count exactly the loads they need (a loop
  // over batches would drain the weight ring too).
  u32x4* xs = reinterpret_cast<u32x4*>(smem);
  const int n_xu = (ts1 - ts0) * (kTileK / 8) * M;
  const float inv_m = 1.0f / (float)M;
  auto load_xunit = [&](int u) {
    int r, m;
    div_small(u, M, inv_m, r, m);
    return *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k0 + 8 * r);
  };
  auto store_xunit = [&](u32x4 q, int u) {
    if constexpr (FMT == 0) {
      // (x0,x1), (x2,x3)/16, (x4,x5), (x6,x7)/16: the order and scale the INT4 masks produce
      q = u32x4{q.x, pk_mul_f16(q.y, kHalfSixteenthPair), q.z, pk_mul_f16(q.w, kHalfSixteenthPair)};
    } else {
      // (x0,x2), (x4,x6), (x1,x3), (x5,x7): the level pairs of bytes 0..3 of a word
      q = u32x4{pair_lo(q.x, q.y), pair_lo(q.z, q.w), pair_hi(q.x, q.y), pair_hi(q.z, q.w)};
    }
    xs[u] = q;
  };

  // Scale block.  Entry (r, j) = the scale (and zero point) words of row r
  // for tile j: GPT = 1, s | z << 16 (NF4: s); GPT = 2, the two groups' s
  // pair, then (INT4) their z pair.  Per-wave blocks (16 rows x the wave's
  // run, rows at pitch sc_pitch, odd, so the 16 rows a lane group reads fall
  // in distinct banks), fetched with row-contiguous loads; or (VS) one block
  // for the workgroup's 16 nwr rows x all KT tiles at row pitch sc_pitch
  // (= 4 mod 32 words), fetched as 16-byte units of 8 groups, each unit of a
  // row one piece of one cache line.
  constexpr int EW = (FMT == 0 && GPT == 2) ? 2 : 1;  // 32-bit words per entry
  uint32_t* sc = reinterpret_cast<uint32_t*>(smem + (size_t)x_bytes) +
                 (VS ? 0 : (size_t)wave * 16 * sc_pitch * EW);
  const int n_se = 16 * cnt;
  const float inv_cnt = 1.0f / (float)max(cnt, 1);
  const size_t srow0 = (size_t)colw * 16 * ng;
  auto load_entry = [&](int e, uint32_t (&v)[EW]) {
    int r, j;
    div_small(e, max(cnt, 1), inv_cnt, r, j);
    const size_t o = srow0 + (size_t)r * ng + (size_t)min(t0 + j, KT - 1) * GPT;  // a wave without tiles still loads
    if constexpr (GPT == 1) {
      v[0] = (uint32_t)scale[o] | (FMT == 0 ? (uint32_t)zero[o] << 16 : 0u);
    } else {
      v[0] = *reinterpret_cast<const uint32_t*>(scale + o);
      if constexpr (EW == 2) v[1] = *reinterpret_cast<const uint32_t*>(zero + o);
    }
  };
  auto store_entry = [&](int e, const uint32_t (&v)[EW]) {
    int r, j;
    div_small(e, max(cnt, 1), inv_cnt, r, j);
#pragma unroll
    for (int w = 0; w < EW; ++w) sc[(r * sc_pitch + j) * EW + w] = v[w];
  };
  // VS: unit u = r * upr + c holds groups 8c .. 8c + 7 of workgroup row r
  constexpr int kVU = 2;  // units per thread (the plan guarantees 16 nwr upr <= kVU threads)
  const int upr = ng / 8;
  const float inv_upr = 1.0f / (float)max(upr, 1);
  auto load_vunit = [&](int u, u32x4& vs, u32x4& vz) {
    int r, c;
    div_small(u, upr, inv_upr, r, c);
    const size_t o = (size_t)min(row_wg0 + r, N - 1) * ng + (size_t)c * 8;
    vs = *reinterpret_cast<const u32x4*>(scale + o);
    if constexpr (FMT == 0) vz = *reinterpret_cast<const u32x4*>(zero + o);
  };
  auto store_vunit = [&](int u, const u32x4& vs, const u32x4& vz) {
    int r, c;
    div_small(u, upr, inv_upr, r, c);
    uint32_t* dst = sc + (size_t)r * sc_pitch;
    if constexpr (GPT == 1) {  // tiles 8c .. 8c + 7: s | z << 16
      uint32_t e[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t zw = FMT == 0 ? vz[i] : 0u;
        e[2 * i] = (vs[i] & 0xFFFFu) | (zw << 16);
        e[2 * i + 1] = (vs[i] >> 16) | (zw & 0xFFFF0000u);
      }
      *reinterpret_cast<u32x4*>(dst + 8 * c) = u32x4{e[0], e[1], e[2], e[3]};
      *reinterpret_cast<u32x4*>(dst + 8 * c + 4) = u32x4{e[4], e[5], e[6], e[7]};
    } else if constexpr (EW == 2) {  // tiles 4c .. 4c + 3: s pair, z pair
      *reinterpret_cast<u32x4*>(dst + 8 * c) = u32x4{vs[0], vz[0], vs[1], vz[1]};
      *reinterpret_cast<u32x4*>(dst + 8 * c + 4) = u32x4{vs[2], vz[2], vs[3], vz[3]};
    } else {  // NF4, tiles 4c .. 4c + 3: s pair
      *reinterpret_cast<u32x4*>(dst + 4 * c) = vs;
    }
  };

  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, (uint32_t)((size_t)N * (K / 2)));
  const uint32_t voff = (uint32_t)lane * 16;
  const uint32_t col_base = (uint32_t)colw * (uint32_t)KT;
  auto load_tile = [&](int t) {
    // a wave without tiles (more waves than tiles) still loads: keep it in bounds
    const int tt = __builtin_amdgcn_readfirstlane(min(min(t, t_last), KT - 1));
    return buffer_load16(wrs, voff, (col_base + (uint32_t)tt) * (uint32_t)kTileBytes);
  };

  // ---- 1. loads, oldest first: NF4 table entries, phase 0 activations,
  // scales, then the weight ring (every count is static, so each wait below
  // covers exactly the loads it needs)
  constexpr int kLutPer = FMT == 1 ? 256 / kWave : 1;  // table entries per thread, at most (64 threads)
  uint32_t lutv[kLutPer];
  if constexpr (FMT == 1) {
#pragma unroll
    for (int i = 0; i < kLutPer; ++i) {
      const int e = min(tid + i * nthr, 255);
      lutv[i] = (uint32_t)float_to_half_bits(nf4_level(e & 15)) |
                ((uint32_t)float_to_half_bits(nf4_level(e >> 4)) << 16);
    }
  }
  // (indices past the end are clamped: the loads stay unconditional, only the
  // stores are predicated)
  u32x4 xb[XU];
#pragma unroll
  for (int i = 0; i < XU; ++i) xb[i] = load_xunit(min(tid + i * nthr, n_xu - 1));
  constexpr int kSEw = VS ? 1 : kSE;
  uint32_t se[kSEw][EW];
  u32x4 vsv[VS ? kVU : 1], vzv[VS ? kVU : 1];
  if constexpr (VS) {
    const int n_vu = 16 * nwr * upr;
#pragma unroll
    for (int i = 0; i < kVU; ++i) load_vunit(min(tid + i * nthr, n_vu - 1), vsv[i], vzv[i]);
  } else {
#pragma unroll
    for (int i = 0; i < kSE; ++i) load_entry(min(lane + i * kWave, max(n_se, 1) - 1), se[i]);
  }
  u32x4 ring[R];
#pragma unroll
  for (int d = 0; d < R; ++d) ring[d] = load_tile(t0 + d);

  // ---- 2. LDS stores as the data arrive
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int u = tid + i * nthr;
    if (u < n_xu) store_xunit(xb[i], u);
  }
  if constexpr (VS) {
    const int n_vu = 16 * nwr * upr;
#pragma unroll
    for (int i = 0; i < kVU; ++i) {
      const int u = tid + i * nthr;
      if (u < n_vu) store_vunit(u, vsv[i], vzv[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSE; ++i) {
      const int e = lane + i * kWave;
      if (e < n_se) store_entry(e, se[i]);
    }
  }
  if constexpr (FMT == 1) {
#pragma unroll
    for (int i = 0; i < kLutPer; ++i) {
      const int e = tid + i * nthr;
      if (e < 256) {
#pragma unroll
        for (int j = 0; j < LC; j += 4) {
          // copies in a lane-rotated order: consecutive entries at one copy
          // would all fall on the same banks
          const int c = (j + 4 * (e % (LC / 4))) % LC;
          *reinterpret_cast<u32x4*>(&lut[e * LC + c]) = u32x4{lutv[i], lutv[i], lutv[i], lutv[i]};
        }
      }
    }
  }
  __syncthreads();

  f32x4 C[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) C[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  int mrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) mrow[t] = ONE ? 0 : TM == 2 ? min(ln >> 2, M - 1) : min(t * 16 + ln, M - 1);
  // INT4: the group's activation sum per token, as a product with constant B
  // (1 for the even pairs, 16 for the pre-scaled odd pairs)
  // (held in VGPRs for the whole run: opaque to the compiler, which would
  // otherwise rebuild the operand from scalar registers for every tile)
  u32x4 kSumB;
  asm volatile("v_mov_b32 %0, 0x3C003C00" : "=v"(kSumB[0]));
  asm volatile("v_mov_b32 %0, 0x4C004C00" : "=v"(kSumB[1]));
  kSumB[2] = kSumB[0];
  kSumB[3] = kSumB[1];
  // the lane's row of the scale block, at the wave's first tile
  const uint32_t* sc_row = VS ? sc + (size_t)(wr * 16 + ln) * sc_pitch + (size_t)t0 * EW
                              : sc + (size_t)ln * sc_pitch * EW;
  const uint32_t* lut_c = lut + lane % LC;
  const uint32_t lane4 = (uint32_t)lane * 4u;
  const int xstride = ONE ? 1 : M;

  // products of tile ci of the wave's run
  auto compute_tile = [&](const u32x4& wv, int ci) {
    uint32_t sz[EW];
#pragma unroll
    for (int w = 0; w < EW; ++w) sz[w] = sc_row[ci * EW + w];
    const uint32_t s_word = sz[0];
    const uint32_t z_word = EW == 2 ? sz[EW - 1] : (sz[0] >> 16);
    u32x4 B[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = wv[w];
      if constexpr (FMT == 0) {
        const uint32_t as = a >> 8;
        B[w] = u32x4{a & 0x000F000Fu, a & 0x00F000F0u, as & 0x000F000Fu, as & 0x00F000F0u};
      } else {
        B[w] = u32x4{lut_pair<LC, 0>(lut, lut_c, lane4, a), lut_pair<LC, 1>(lut, lut_c, lane4, a),
                     lut_pair<LC, 2>(lut, lut_c, lane4, a), lut_pair<LC, 3>(lut, lut_c, lane4, a)};
      }
    }
    const int tl = t0 - ts0 + ci;  // tile index within the slice
    const u32x4* xa = xs + (size_t)(tl * 16 + kb) * xstride;  // + (4 w) * M + m
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = gi * WPG; w < (gi + 1) * WPG; ++w) acc = mfma_f16(xa[(4 * w) * xstride + mrow[t]], B[w], acc);
        constexpr int NI = TM != 0 ? 1 : 4;  // accumulator elements that hold tokens
        if constexpr (FMT == 0) {
          // y += (s 2^24) sum x q 2^-24 - (s z) sum x
          f32x4 sx = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = gi * WPG; w < (gi + 1) * WPG; ++w) sx = mfma_f16(xa[(4 * w) * xstride + mrow[t]], kSumB, sx);
          const float sv = half_bits_to_float((uint16_t)(GPT == 1 ? s_word : s_word >> (16 * gi)));
          const float zv = half_bits_to_float((uint16_t)(GPT == 1 ? z_word : z_word >> (16 * gi)));
          const float ex = sv * 16777216.0f, ey = -sv * zv;  // codes enter as q * 2^-24
#pragma unroll
          for (int i = 0; i < NI; ++i) C[t][i] = fmaf(ex, acc[i], fmaf(ey, sx[i], C[t][i]));
        } else {
          const float sv = half_bits_to_float((uint16_t)(GPT == 1 ? s_word : s_word >> (16 * gi)));
#pragma unroll
          for (int i = 0; i < NI; ++i) C[t][i] = fmaf(sv, acc[i], C[t][i]);
        }
      }
    }
  };

  // ---- 3. the run.  A ring slot is consumed before its refill is issued, so
  // the refill lands in the same registers (moving a register whose load is
  // still in flight would make the wave wait for it, draining the ring).
  if (cnt > 0) {
    const int cnt_pad = (cnt + R - 1) / R * R;
    int base = 0;
    for (; base + R < cnt_pad; base += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) {
        const int ci = base + d;
        if (ci < cnt) compute_tile(ring[d], ci);
        ring[d] = load_tile(t0 + ci + R);
      }
    }
#pragma unroll
    for (int d = 0; d < R; ++d) {  // last block: no refill
      const int ci = base + d;
      if (ci < cnt) compute_tile(ring[d], ci);
    }
  }
  __syncthreads();

  // ---- cross-wave reduction (over wk) through LDS, reusing the staging area
  gemv_finish<MT, TM>(C, reinterpret_cast<float*>(smem), wave, lane, nwr, nwk, row_wg0, M, N, y, partial);
}

// Direct variant.  Each wave owns C tile columns (16 C weight rows) and a run
// of K tiles; the workgroup's waves split K between them and add their
// results through LDS at the end.  The activations are read from memory (L2,
// where all workgroups find them) straight into matrix-core A operands: no
// staging and no barrier before the products.  One set of A operands serves C
// weight tiles, and for INT4 the group's activation sum too, so the operand
// traffic per weight byte falls with C.  The unpacked INT4 pairs all carry
// the same 2^-24 (the odd pairs are shifted down rather than the
// activations pre-scaled); for NF4 the activation pairs are permuted in
// registers to the byte order of the level pairs.
// VS: as in the staged kernel, one scale block for the workgroup's 16 C rows
// and all of K, fetched with 16-byte loads.
// XL: the activations of a tile are loaded whole rows at a time (load j:
// rows 4 j .. 4 j + 3 of the token tile, 256 bytes each, so each load
// touches 8 cache lines instead of the 16 half-used lines of the operand
// order) and pass through a 4 KB LDS area of the wave's own, written in that
// order and read back in the operand order (chunk c of row r at slot
// c ^ r: both sides free of bank conflicts).  The wave's LDS accesses
// complete in order, so no barrier is involved.
template <int FMT, int LB, int MT, int C, int R, bool VS, bool XL, int LC>
__global__ __launch_bounds__(kGemvMaxThreads) void gemv_direct_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    float* __restrict__ partial, int sc_pitch, int xl_off) {
  constexpr int G = 8 * LB;
  constexpr int GPT = kTileK / G;
  constexpr int WPG = 4 / GPT;
  constexpr int EW = (FMT == 0 && GPT == 2) ? 2 : 1;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t lut[FMT == 1 ? 256 * LC : 1];

  const int lane = threadIdx.x % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // = the K wave
  const int nwk = blockDim.x / kWave;
  const int ln = lane % 16;
  const int kb = lane / 16;
  const int ng = K / G;
  const int KT = K / kTileK;
  const int ncol = N / 16;
  const int col0 = blockIdx.x * C;
  const int S = gridDim.y;
  const int ks = blockIdx.y;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;

  const int ts0 = (int)((long)KT * ks / S), ts1 = (int)((long)KT * (ks + 1) / S);
  const int t0 = ts0 + (int)((long)(ts1 - ts0) * wave / nwk);
  const int cnt = ts0 + (int)((long)(ts1 - ts0) * (wave + 1) / nwk) - t0;
  const int t_last = t0 + max(cnt, 1) - 1;
  int colc[C];  // a group past the last column re-reads it and stores nothing
#pragma unroll
  for (int c = 0; c < C; ++c) colc[c] = min(col0 + c, ncol - 1);

  // scale block of this wave: entry (c, r, j) = column c, row r, tile t0 + j;
  // VS: of the workgroup, entry (c, r, tile) at row 16 c + r, pitch sc_pitch
  uint32_t* sc = reinterpret_cast<uint32_t*>(smem) + (VS ? 0 : (size_t)wave * C * 16 * sc_pitch * EW);
  const int n_se = C * 16 * cnt;
  const float inv_cnt = 1.0f / (float)max(cnt, 1);
  auto load_entry = [&](int e, uint32_t (&v)[EW]) {
    int cr, j;
    div_small(e, max(cnt, 1), inv_cnt, cr, j);
    const int c = cr / 16, r = cr % 16;
    const size_t o = (size_t)(min(col0 + c, ncol - 1) * 16 + r) * ng + (size_t)min(t0 + j, KT - 1) * GPT;
    if constexpr (GPT == 1) {
      v[0] = (uint32_t)scale[o] | (FMT == 0 ? (uint32_t)zero[o] << 16 : 0u);
    } else {
      v[0] = *reinterpret_cast<const uint32_t*>(scale + o);
      if constexpr (EW == 2) v[1] = *reinterpret_cast<const uint32_t*>(zero + o);
    }
  };

  constexpr int kVU = 2;  // VS units per thread (the plan guarantees 16 C upr <= kVU threads)
  const int upr = ng / 8;
  const float inv_upr = 1.0f / (float)max(upr, 1);
  auto load_vunit = [&](int u, u32x4& vs, u32x4& vz) {
    int r, cg;
    div_small(u, upr, inv_upr, r, cg);
    const size_t o = (size_t)(min(col0 + r / 16, ncol - 1) * 16 + r % 16) * ng + (size_t)cg * 8;
    vs = *reinterpret_cast<const u32x4*>(scale + o);
    if constexpr (FMT == 0) vz = *reinterpret_cast<const u32x4*>(zero + o);
  };
  auto store_vunit = [&](int u, const u32x4& vs, const u32x4& vz) {
    int r, cg;
    div_small(u, upr, inv_upr, r, cg);
    uint32_t* dst = sc + (size_t)r * sc_pitch;
    if constexpr (GPT == 1) {  // tiles 8 cg .. 8 cg + 7: s | z << 16
      uint32_t e[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t zw = FMT == 0 ? vz[i] : 0u;
        e[2 * i] = (vs[i] & 0xFFFFu) | (zw << 16);
        e[2 * i + 1] = (vs[i] >> 16) | (zw & 0xFFFF0000u);
      }
      *reinterpret_cast<u32x4*>(dst + 8 * cg) = u32x4{e[0], e[1], e[2], e[3]};
      *reinterpret_cast<u32x4*>(dst + 8 * cg + 4) = u32x4{e[4], e[5], e[6], e[7]};
    } else if constexpr (EW == 2) {  // tiles 4 cg .. 4 cg + 3: s pair, z pair
      *reinterpret_cast<u32x4*>(dst + 8 * cg) = u32x4{vs[0], vz[0], vs[1], vz[1]};
      *reinterpret_cast<u32x4*>(dst + 8 * cg + 4) = u32x4{vs[2], vz[2], vs[3], vz[3]};
    } else {  // NF4, tiles 4 cg .. 4 cg + 3: s pair
      *reinterpret_cast<u32x4*>(dst + 4 * cg) = vs;
    }
  };

  // ring slot: the lane's 16 bytes of C weight tiles and its A operands
  struct Slot {
    u32x4 w[C];
    u32x4 a[4][MT];
  };
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, (uint32_t)((size_t)N * (K / 2)));
  const uint32_t voff = (uint32_t)lane * 16;
  // operand order: lane (ln, kb) reads row ln, chunk 4 w + kb of word w;
  // XL: load j gives lane (ln, kb) row 4 j + kb, chunk ln.  Buffer loads:
  // the lane's byte offset in a VGPR, the tile's (tt * 256) in an SGPR, so
  // no per-load 64-bit address arithmetic.
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, (uint32_t)((size_t)M * K * 2));
  uint32_t xoff[XL ? 4 : 1][MT];
#pragma unroll
  for (int j = 0; j < (XL ? 4 : 1); ++j)
#pragma unroll
    for (int m = 0; m < MT; ++m)
      xoff[j][m] = XL ? (uint32_t)min(m * 16 + 4 * j + kb, M - 1) * (uint32_t)K * 2u + (uint32_t)ln * 16u
                      : (uint32_t)min(m * 16 + ln, M - 1) * (uint32_t)K * 2u + (uint32_t)kb * 16u;
  auto load_slot = [&](Slot& sl, int t) {
    const int tt = __builtin_amdgcn_readfirstlane(min(min(t, t_last), KT - 1));
#pragma unroll
    for (int c = 0; c < C; ++c)
      sl.w[c] = buffer_load16(wrs, voff, ((uint32_t)colc[c] * (uint32_t)KT + (uint32_t)tt) * (uint32_t)kTileBytes);
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int m = 0; m < MT; ++m)
        sl.a[w][m] = XL ? buffer_load16_cached(xrs, xoff[w][m], (uint32_t)tt * 256u)
                        : buffer_load16_cached(xrs, xoff[0][m] + 64u * (uint32_t)w, (uint32_t)tt * 256u);
  };
  unsigned char* const xs = smem + xl_off + (size_t)wave * MT * 4096;  // XL: this wave's area

  // ---- prologue: table entries, scale entries, then the ring
  constexpr int kLutPer = FMT == 1 ? 256 / kWave : 1;
  uint32_t lutv[kLutPer];
  if constexpr (FMT == 1) {
#pragma unroll
    for (int i = 0; i < kLutPer; ++i) {
      const int e = min(tid + i * nthr, 255);
      lutv[i] = (uint32_t)float_to_half_bits(nf4_level(e & 15)) |
                ((uint32_t)float_to_half_bits(nf4_level(e >> 4)) << 16);
    }
  }
  constexpr int kSEw = VS ? 1 : kSEDirect;
  uint32_t se[kSEw][EW];
  u32x4 vsv[VS ? kVU : 1], vzv[VS ? kVU : 1];
  if constexpr (VS) {
    const int n_vu = C * 16 * upr;
#pragma unroll
    for (int i = 0; i < kVU; ++i) load_vunit(min(tid + i * nthr, n_vu - 1), vsv[i], vzv[i]);
  } else {
#pragma unroll
    for (int i = 0; i < kSEDirect; ++i) load_entry(min(lane + i * kWave, max(n_se, 1) - 1), se[i]);
  }
  Slot ring[R];
#pragma unroll
  for (int d = 0; d < R; ++d) {
    load_slot(ring[d], t0 + d);
    // keep the slots' loads in slot order, as the refills issue them, so the
    // waits in the loop count the same way on entry as in steady state
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (VS) {
    const int n_vu = C * 16 * upr;
#pragma unroll
    for (int i = 0; i < kVU; ++i) {
      const int u = tid + i * nthr;
      if (u < n_vu) store_vunit(u, vsv[i], vzv[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < kSEDirect; ++i) {
      const int e = lane + i * kWave;
      if (e < n_se) {
        int cr, j;
        div_small(e, max(cnt, 1), inv_cnt, cr, j);
#pragma unroll
        for (int w = 0; w < EW; ++w) sc[(cr * sc_pitch + j) * EW + w] = se[i][w];
      }
    }
  }
  if constexpr (FMT == 1) {
#pragma unroll
    for (int i = 0; i < kLutPer; ++i) {
      const int e = tid + i * nthr;
      if (e < 256) {
#pragma unroll
        for (int j = 0; j < LC; j += 4) {
          // copies in a lane-rotated order: consecutive entries at one copy
          // would all fall on the same banks
          const int c = (j + 4 * (e % (LC / 4))) % LC;
          *reinterpret_cast<u32x4*>(&lut[e * LC + c]) = u32x4{lutv[i], lutv[i], lutv[i], lutv[i]};
        }
      }
    }
    if constexpr (!VS) __syncthreads();  // the table is shared; the scale block is the wave's own
  }
  if constexpr (VS) __syncthreads();  // the workgroup's scale block (and the NF4 table) are shared

  f32x4 acc_c[C][MT];
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m) acc_c[c][m] = f32x4{0.f, 0.f, 0.f, 0.f};
  // held in VGPRs for the whole run (opaque to the compiler, which would
  // otherwise rebuild the operand from scalar registers for every step)
  u32x4 kOnes;
  asm volatile("v_mov_b32 %0, 0x3C003C00" : "=v"(kOnes[0]));
  kOnes[1] = kOnes[2] = kOnes[3] = kOnes[0];
  const uint32_t* lut_c = lut + lane % LC;
  const uint32_t lane4 = (uint32_t)lane * 4u;

  auto compute = [&](Slot& sl, int ci) {
    if constexpr (XL) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          *reinterpret_cast<u32x4*>(xs + m * 4096 + (4 * j + kb) * 256 + ((ln ^ (4 * j + kb)) << 4)) = sl.a[j][m];
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int m = 0; m < MT; ++m)
          sl.a[w][m] = *reinterpret_cast<const u32x4*>(xs + m * 4096 + ln * 256 + (((4 * w + kb) ^ ln) << 4));
    }
    if constexpr (FMT == 1) {
      // activation pairs in the order of the level pairs of bytes 0..3: (x0,x2), (x4,x6), (x1,x3), (x5,x7)
#pragma unroll
      for (int w = 0; w < 4; ++w)
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const u32x4 q = sl.a[w][m];
          sl.a[w][m] = u32x4{pair_lo(q.x, q.y), pair_lo(q.z, q.w), pair_hi(q.x, q.y), pair_hi(q.z, q.w)};
        }
    }
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      f32x4 sx[MT];
      if constexpr (FMT == 0) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          sx[m] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = gi * WPG; w < (gi + 1) * WPG; ++w) sx[m] = mfma_f16(sl.a[w][m], kOnes, sx[m]);
        }
      }
#pragma unroll
      for (int c = 0; c < C; ++c) {
        uint32_t sz[EW];
#pragma unroll
        for (int w = 0; w < EW; ++w)
          sz[w] = VS ? sc[(size_t)(c * 16 + ln) * sc_pitch + (size_t)(t0 + ci) * EW + w]
                     : sc[((c * 16 + ln) * sc_pitch + ci) * EW + w];
        const float sv = GPT == 1 ? half_bits_to_float((uint16_t)(sz[0] & 0xFFFFu))
                                  : half_bits_to_float((uint16_t)(sz[0] >> (16 * gi)));
        u32x4 B[WPG];
#pragma unroll
        for (int wi = 0; wi < WPG; ++wi) {
          const uint32_t a = sl.w[c][gi * WPG + wi];
          if constexpr (FMT == 0) {
            B[wi] = u32x4{a & 0x000F000Fu, (a >> 4) & 0x000F000Fu, (a >> 8) & 0x000F000Fu, (a >> 12) & 0x000F000Fu};
          } else {
            B[wi] = u32x4{lut_pair<LC, 0>(lut, lut_c, lane4, a), lut_pair<LC, 1>(lut, lut_c, lane4, a),
                          lut_pair<LC, 2>(lut, lut_c, lane4, a), lut_pair<LC, 3>(lut, lut_c, lane4, a)};
          }
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int wi = 0; wi < WPG; ++wi) acc = mfma_f16(sl.a[gi * WPG + wi][m], B[wi], acc);
          if constexpr (FMT == 0) {
            const uint32_t zw = EW == 2 ? sz[EW - 1] : (sz[0] >> 16);
            const float zv = GPT == 1 ? half_bits_to_float((uint16_t)(zw & 0xFFFFu))
                                      : half_bits_to_float((uint16_t)(zw >> (16 * gi)));
            const float ex = sv * 16777216.0f, ey = -sv * zv;  // codes enter as q * 2^-24
#pragma unroll
            for (int i = 0; i < 4; ++i) acc_c[c][m][i] = fmaf(ex, acc[i], fmaf(ey, sx[m][i], acc_c[c][m][i]));
          } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc_c[c][m][i] = fmaf(sv, acc[i], acc_c[c][m][i]);
          }
        }
      }
    }
  };

  if (cnt > 0) {
    const int cnt_pad = (cnt + R - 1) / R * R;
    int base = 0;
    for (; base + R < cnt_pad; base += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) {
        const int ci = base + d;
        if (ci < cnt) compute(ring[d], ci);
        load_slot(ring[d], t0 + ci + R);
      }
    }
#pragma unroll
    for (int d = 0; d < R; ++d) {
      const int ci = base + d;
      if (ci < cnt) compute(ring[d], ci);
    }
  }

  // ---- sum over the K waves through LDS (the scale blocks are dead by now)
  __syncthreads();
  constexpr int kT = MT * 256;  // one column's outputs
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int c = 0; c < C; ++c)
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[(wave * C + c) * kT + (m * 4 + i) * 64 + lane] = acc_c[c][m][i];
  __syncthreads();
  for (int e = tid; e < C * kT; e += nthr) {
    const int c = e / kT;
    const int el = e - c * kT;
    const int l = el % 64;
    const int i = (el / 64) % 4;
    const int t = el / 256;
    const int m = t * 16 + 4 * (l / 16) + i;
    if (m >= M || col0 + c >= ncol) continue;
    const int n = (col0 + c) * 16 + l % 16;
    float sum = 0.f;
    for (int w2 = 0; w2 < nwk; ++w2) sum += red[(w2 * C + c) * kT + el];
    if (S == 1)
      y[(size_t)m * N + n] = float_to_half_bits(sum);
    else
      partial[((size_t)ks * M + m) * N + n] = sum;
  }
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

constexpr int kGemvLdsTarget = 78 * 1024;   // two workgroups per CU (160 KB of LDS)
constexpr int kGemvLdsOne = 150 * 1024;     // one workgroup per CU (static LDS included)
constexpr int kCUs = 256;
constexpr int kLutBytes = 256 * kLutCopies * 4;
constexpr int kLutBytesWide = 256 * kLutCopiesWide * 4;

}  // namespace

// Direct variant: C columns per wave, nwk K waves per workgroup, K split
// over workgroups only while the grid is short of about 2048 waves or a run
// would exceed the scale block.
void plan_direct(GemvPlan& c, int M, int K, int N, int G, int fmt) {
  const int KT = K / kTileK;
  const int gpt = kTileK / G;
  const int max_waves = kGemvMaxThreads / kWave;
  c.kind = 1;
  c.ring = M <= 16 ? 4 : 2;
  c.mt = M <= 16 ? 1 : 2;
  c.nwr = 1;
  // Measured on MI355X (K x N = 8192 x 8192, 8192 x 28672, 28672 x 8192):
  // two tile columns and eight K waves per workgroup, except four columns
  // (each activation operand serving twice the weight rows) from M = 9 on for
  // layers of 2^27 weights or more, and four K waves at M <= 8 once the grid
  // has 512 or more column pairs.
  c.cols = 2;
  c.nwk = 8;
  if (M > 8 && (long)N * K >= (1L << 27)) {
    c.cols = 4;
  } else if (M <= 8 && N / 32 >= 512) {
    c.nwk = 4;
  }
  const int cols = env_int("W4_GEMV_C", 0);
  const int nwk = env_int("W4_GEMV_NWK", 0);
  const int s = env_int("W4_GEMV_S", 0);
  if (cols == 1 || cols == 2 || cols == 4) c.cols = cols;
  if (nwk >= 1 && nwk <= max_waves) c.nwk = nwk;
  const int groups = (N / 16 + c.cols - 1) / c.cols;
  c.s = 1;
  if (s >= 1 && s <= KT) {
    c.s = s;
  } else {
    while ((long)groups * c.s * c.nwk < 2048 && KT / (c.s * 2 * c.nwk) >= 4) c.s *= 2;
  }
  const int max_run = kSEDirect * kWave / (16 * c.cols);
  while (((KT + c.s - 1) / c.s + c.nwk - 1) / c.nwk > max_run) ++c.s;
  const int run = ((KT + c.s - 1) / c.s + c.nwk - 1) / c.nwk;
  const int ew = (fmt == 0 && gpt == 2) ? 2 : 1;
  c.sc_pitch = run | 1;
  c.x_bytes = 0;
  c.xu = 0;
  const long sc_bytes = (long)c.nwk * c.cols * 16 * c.sc_pitch * ew * 4;
  const long red = (long)c.nwk * c.cols * c.mt * 256 * 4;
  c.lds_bytes = (size_t)(sc_bytes > red ? sc_bytes : red);
  c.row_blocks = groups;
  // the workgroup's scale block with 16-byte loads (as in the staged kernel);
  // it and the reduction area are never live together
  const int ng = K / G;
  c.vs = 0;
  if (c.s == 1 && ng % 8 == 0 && 16L * c.cols * (ng / 8) <= 2L * c.nwk * kWave) {
    const int pitch = (KT * ew + 31) / 32 * 32 + 4;
    const long vs_bytes = 16L * c.cols * pitch * 4;
    if (vs_bytes <= sc_bytes + 8 * 1024) {
      c.vs = 1;
      c.sc_pitch = pitch;
      c.lds_bytes = (size_t)(vs_bytes > red ? vs_bytes : red);
    }
  }
  // activations whole rows at a time through a per-wave LDS area (4 KB per
  // token tile) after the scale block or reduction area, when it fits the
  // budget.  Measured on MI355X against the operand-order loads: M = 32 (two
  // token tiles) 4-10 % faster on the MLP layers, M = 16 INT4 2-3 % faster,
  // NF4 at M = 16 even, M = 8 up to 10 % slower (the LDS round trip's
  // latency outweighs the halved cache-line count there).
  c.xl = 0;
  c.xl_off = 0;
  const size_t xl_off = (c.lds_bytes + 255) / 256 * 256;
  const size_t xl_bytes = xl_off + (size_t)c.nwk * c.mt * 4096;
  const int xl = env_int("W4_GEMV_XL", -1);
  const bool xl_default = M > 16 || (M == 16 && fmt == 0);
  if ((xl < 0 ? xl_default : xl != 0) && xl_bytes <= gemv_lds_budget(fmt)) {
    c.xl = 1;
    c.xl_off = (int)xl_off;
    c.lds_bytes = xl_bytes;
  }
  (void)M;
}

GemvPlan plan_gemv(int M, int K, int N, int G, int fmt) {
  GemvPlan c;
  c.xl = 0;
  c.xl_off = 0;
  const int KT = K / kTileK;  // tiles per 16-row column
  const int gpt = kTileK / G;
  const int max_waves = kGemvMaxThreads / kWave;
  c.mt = M <= 16 ? 1 : 2;
  // Measured on MI355X (K = N = 8192, 8192 x 28672, 28672 x 8192, both
  // formats): two 16-row tile columns per workgroup with four K waves up to
  // M = 8 (the staged activations serve twice the weight rows); beyond, eight
  // columns with one K wave each, so that the activations, which outweigh the
  // weights per K position from M = 8 on, are staged once per 128 rows.  On
  // layers of 2^27 weights or more (the MLP matrices): one column at M <= 2,
  // eight columns and one K wave from M = 3 on.  K is split over workgroups
  // (fp32 partials and a second kernel) while the grid holds fewer than about
  // 2048 waves, or while the slice's activations would not fit one staging
  // batch or the LDS.
  const bool large = (long)N * K >= (1L << 27);
  c.nwr = M <= 8 ? 2 : 8;
  c.nwk = M <= 8 ? 4 : 1;
  if (large && M <= 2) c.nwr = 1;
  if (large && M > 2) {
    c.nwr = 8;
    c.nwk = 1;
  }
  const int nwr = env_int("W4_GEMV_NWR", 0);
  const int nwk = env_int("W4_GEMV_NWK", 0);
  const int s = env_int("W4_GEMV_S", 0);
  if (nwr >= 1 && nwr <= max_waves) c.nwr = nwr;
  if (nwk >= 1 && nwk <= max_waves) c.nwk = nwk;
  if (c.nwr * c.nwk > max_waves) c.nwk = max(1, max_waves / c.nwr);
  c.row_blocks = (N + 16 * c.nwr - 1) / (16 * c.nwr);
  c.s = 1;
  if (s >= 1 && s <= KT) {
    c.s = s;
  } else {
    const int want_waves = 2048;
    while (c.row_blocks * c.s * c.nwr * c.nwk < want_waves && KT / (c.s * 2 * c.nwk) >= 8) c.s *= 2;
  }
  const int ew = (fmt == 0 && gpt == 2) ? 2 : 1;  // 32-bit words per scale entry
  for (;;) {
    const int slice_max = (KT + c.s - 1) / c.s;
    const int nthr = c.nwr * c.nwk * kWave;
    const int run = (slice_max + c.nwk - 1) / c.nwk;
    const long n_xu = (long)slice_max * (kTileK / 8) * M;
    if (n_xu > (long)kXUMax * nthr || run > kMaxRun) {
      if (c.nwr * c.nwk * 2 <= max_waves) c.nwk *= 2;
      else if (c.s < KT) ++c.s;
      else break;  // not reached: one tile per slice always fits
      continue;
    }
    c.sc_pitch = run | 1;
    c.x_bytes = (int)(n_xu * 16);
    c.xu = n_xu <= (long)kXUSmall * nthr ? kXUSmall : kXUMax;
    const long sc_bytes = (long)c.nwr * c.nwk * 16 * c.sc_pitch * ew * 4;
    const long red = (long)c.nwr * c.nwk * c.mt * 256 * 4;
    const long need = c.x_bytes + sc_bytes;
    c.lds_bytes = (size_t)(need > red ? need : red);
    const long wgs = (long)((N + 16 * c.nwr - 1) / (16 * c.nwr)) * c.s;
    const long target = (wgs > kCUs ? kGemvLdsTarget : kGemvLdsOne) - (fmt == 1 ? kLutBytes : 0);
    if ((long)c.lds_bytes <= target || c.s >= KT) break;
    ++c.s;
  }
  c.row_blocks = (N + 16 * c.nwr - 1) / (16 * c.nwr);
  // the workgroup's scale block with 16-byte loads: K not split, K / G a
  // multiple of 8 (whole units per row), at most kVU units per thread, and
  // no more LDS than the per-wave blocks
  const int ng = K / G;
  c.vs = 0;
  if (c.s == 1 && ng % 8 == 0 && 16L * c.nwr * (ng / 8) <= 2L * c.nwr * c.nwk * kWave) {
    const int pitch = (KT * ew + 31) / 32 * 32 + 4;  // 16-byte rows, 4 mod 32 words
    const long vs_bytes = 16L * c.nwr * pitch * 4;
    const long ws_bytes = (long)c.nwr * c.nwk * 16 * c.sc_pitch * ew * 4;
    if (vs_bytes <= ws_bytes + 8 * 1024) {
      c.vs = 1;
      c.sc_pitch = pitch;
      const long red = (long)c.nwr * c.nwk * c.mt * 256 * 4;
      const long need = c.x_bytes + vs_bytes;
      c.lds_bytes = (size_t)(need > red ? need : red);
    }
  }
  c.kind = 0;
  c.cols = 1;
  c.ring = kRing;
  const int ring = env_int("W4_GEMV_RING", 0);
  if (c.mt == 1 && (ring == 4 || ring == 8 || ring == 16)) c.ring = ring;
  // Measured on MI355X (K = N = 8192): the staged kernel is faster up to M =
  // 4, the direct one (two columns per wave, eight K waves) beyond, where the
  // staged activations would outweigh the weights a workgroup streams.
  const int kind = env_int("W4_GEMV_KIND", -1);
  if (kind == 1 || (kind != 0 && M > kDirectFromM)) plan_direct(c, M, K, N, G, fmt);
  c.ws_bytes = c.s > 1 ? (size_t)c.s * M * N * sizeof(float) : 0;
  // NF4: the 64-copy table where the plan runs one workgroup per CU (one
  // token tile, the default ring), its LDS leaves room for it and the layer
  // is large enough (2^25 weights or more) to repay filling 64 KB per
  // workgroup; the plan itself is the one chosen for the 16-copy table
  c.lut = kLutCopies;
  if (fmt == 1 && c.mt == 1 && c.ring == kRing && (long)c.row_blocks * c.s <= kCUs && (long)N * K >= (1L << 25) &&
      c.lds_bytes + kLutBytesWide <= (size_t)kGemvLdsOne && env_int("W4_GEMV_LUT", kLutCopiesWide) == kLutCopiesWide)
    c.lut = kLutCopiesWide;
  return c;
}

size_t gemv_lds_budget(int fmt) { return (size_t)(kGemvLdsOne - (fmt == 1 ? kLutBytes : 0)); }
size_t gemv_static_lds(int fmt) { return fmt == 1 ? (size_t)kLutBytes : 4; }
size_t gemv_plan_static_lds(const GemvPlan& c, int fmt) { return fmt == 1 ? (size_t)256 * c.lut * 4 : 4; }
size_t gemv_plan_lds_budget(const GemvPlan& c, int fmt) {
  return (size_t)kGemvLdsOne - (fmt == 1 ? (size_t)256 * c.lut * 4 : 0);
}
int gemv_plan_threads(const GemvPlan& c) { return (c.kind == 1 ? 1 : c.nwr) * c.nwk * kWave; }

int check_gemv_plan(const GemvPlan& c, int fmt) {
  if (gemv_plan_threads(c) > kGemvMaxThreads)  // the kernels are built for at most this many threads
    return fail(-1 /* W4_EINVAL */, "w4_gemv: plan with %d x %d waves exceeds the kernel's %d threads",
                c.kind == 1 ? 1 : c.nwr, c.nwk, kGemvMaxThreads);
  if (c.lds_bytes > gemv_plan_lds_budget(c, fmt))
    return fail(-2 /* W4_EUNSUPPORTED */, "w4_gemv: plan needs %zu bytes of LDS (at most %zu)", c.lds_bytes,
                gemv_plan_lds_budget(c, fmt));
  return 0;
}

namespace {

template <int FMT, int LB, int MT, int XU, int R, int TM, bool VS, int LC>
int launch_t1(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
              const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  if (const int bad = check_gemv_plan(c, FMT)) return bad;
  const dim3 block(c.nwr * c.nwk * kWave);
  const dim3 grid((unsigned)c.row_blocks, (unsigned)c.s);
  float* partial = c.s > 1 ? static_cast<float*>(ws) : nullptr;
  // the plan's one-workgroup budget; the NF4 table is static LDS on top
  const int st = allow_dynamic_lds(reinterpret_cast<const void*>(&gemv_kernel<FMT, LB, MT, XU, R, TM, VS, LC>),
                                   kGemvLdsOne - (FMT == 1 ? 256 * LC * 4 : 0), "w4_gemv");
  if (st != 0) return st;
  hipLaunchKernelGGL((gemv_kernel<FMT, LB, MT, XU, R, TM, VS, LC>), grid, block, c.lds_bytes, s, x, M, K, N, packed, scale, zero,
                     y, partial, c.nwr, c.nwk, c.sc_pitch, c.x_bytes);
  if (c.s > 1) return launch_reduce_partials(partial, c.s, (long)M * N, y, s);
  return check_launch("gemv");
}

template <int FMT, int LB, int MT, int XU, int R, int LC>
int launch_t_lc(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  if constexpr (MT == 1) {
    if (M == 1) {
      if (c.vs) return launch_t1<FMT, LB, 1, XU, R, 1, true, LC>(c, x, M, K, N, packed, scale, zero, y, ws, s);
      return launch_t1<FMT, LB, 1, XU, R, 1, false, LC>(c, x, M, K, N, packed, scale, zero, y, ws, s);
    }
    if (M <= 4) {
      if (c.vs) return launch_t1<FMT, LB, 1, XU, R, 2, true, LC>(c, x, M, K, N, packed, scale, zero, y, ws, s);
      return launch_t1<FMT, LB, 1, XU, R, 2, false, LC>(c, x, M, K, N, packed, scale, zero, y, ws, s);
    }
  }
  if (c.vs) return launch_t1<FMT, LB, MT, XU, R, 0, true, LC>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  return launch_t1<FMT, LB, MT, XU, R, 0, false, LC>(c, x, M, K, N, packed, scale, zero, y, ws, s);
}

template <int FMT, int LB, int MT, int XU, int R>
int launch_t(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
             const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  if constexpr (FMT == 1 && MT == 1 && R == kRing)
    if (c.lut == kLutCopiesWide)
      return launch_t_lc<FMT, LB, MT, XU, R, kLutCopiesWide>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  return launch_t_lc<FMT, LB, MT, XU, R, kLutCopies>(c, x, M, K, N, packed, scale, zero, y, ws, s);
}

template <int FMT, int LB, int MT, int C, bool VS, bool XL, int LC>
int launch_direct1_lc(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                   const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  constexpr int R = MT == 1 ? 4 : 2;
  const dim3 block(c.nwk * kWave);
  const dim3 grid((unsigned)c.row_blocks, (unsigned)c.s);
  float* partial = c.s > 1 ? static_cast<float*>(ws) : nullptr;
  // the one-workgroup budget (the NF4 table is static LDS on top), reserved
  // once per instantiation: beyond 64 KB of dynamic LDS a launch needs it
  const int budget = kGemvLdsOne - (FMT == 1 ? 256 * LC * 4 : 0);
  if (const int bad = check_gemv_plan(c, FMT)) return bad;
  const int st = allow_dynamic_lds(reinterpret_cast<const void*>(&gemv_direct_kernel<FMT, LB, MT, C, R, VS, XL, LC>),
                                   budget, "w4_gemv");
  if (st != 0) return st;
  hipLaunchKernelGGL((gemv_direct_kernel<FMT, LB, MT, C, R, VS, XL, LC>), grid, block, c.lds_bytes, s, x, M, K, N, packed,
                     scale, zero, y, partial, c.sc_pitch, c.xl_off);
  if (c.s > 1) return launch_reduce_partials(partial, c.s, (long)M * N, y, s);
  return check_launch("gemv");
}

template <int FMT, int LB, int MT, int C, bool VS, bool XL>
int launch_direct1(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                   const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  if constexpr (FMT == 1 && MT == 1)
    if (c.lut == kLutCopiesWide)
      return launch_direct1_lc<FMT, LB, MT, C, VS, XL, kLutCopiesWide>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  return launch_direct1_lc<FMT, LB, MT, C, VS, XL, kLutCopies>(c, x, M, K, N, packed, scale, zero, y, ws, s);
}

template <int FMT, int LB, int MT, int C>
int launch_direct(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                  const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  if (c.xl) {
    if (c.vs) return launch_direct1<FMT, LB, MT, C, true, true>(c, x, M, K, N, packed, scale, zero, y, ws, s);
    return launch_direct1<FMT, LB, MT, C, false, true>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  }
  if (c.vs) return launch_direct1<FMT, LB, MT, C, true, false>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  return launch_direct1<FMT, LB, MT, C, false, false>(c, x, M, K, N, packed, scale, zero, y, ws, s);
}

template <int FMT, int LB, int MT>
int launch_direct_c(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                    const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  if (c.cols == 1) return launch_direct<FMT, LB, MT, 1>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  if (c.cols == 4) return launch_direct<FMT, LB, MT, 4>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  return launch_direct<FMT, LB, MT, 2>(c, x, M, K, N, packed, scale, zero, y, ws, s);
}

template <int FMT, int LB>
int launch_mt(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
              const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  if (c.kind == 1) {
    if (c.mt == 1) return launch_direct_c<FMT, LB, 1>(c, x, M, K, N, packed, scale, zero, y, ws, s);
    return launch_direct_c<FMT, LB, 2>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  }
  if (c.mt == 1) {
#define W4_GEMV_STAGED_R(XU)                                                                        \
  switch (c.ring) {                                                                                 \
    case 16: return launch_t<FMT, LB, 1, XU, 16>(c, x, M, K, N, packed, scale, zero, y, ws, s);    \
    case 8: return launch_t<FMT, LB, 1, XU, 8>(c, x, M, K, N, packed, scale, zero, y, ws, s);      \
    default: return launch_t<FMT, LB, 1, XU, kRing>(c, x, M, K, N, packed, scale, zero, y, ws, s); \
  }
    if (c.xu == kXUSmall) W4_GEMV_STAGED_R(kXUSmall)
    W4_GEMV_STAGED_R(kXUMax)
#undef W4_GEMV_STAGED_R
  }
  if (c.xu == kXUSmall) return launch_t<FMT, LB, 2, kXUSmall, kRing>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  return launch_t<FMT, LB, 2, kXUMax, kRing>(c, x, M, K, N, packed, scale, zero, y, ws, s);
}

}  // namespace

int launch_reduce_partials(const float* partial, int S, long MN, uint16_t* y, hipStream_t s) {
  const long threads = (MN + 3) / 4;
  hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, partial, S, MN, y);
  return check_launch("reduce partials");
}

int launch_gemv(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                const uint16_t* scale, const uint16_t* zero, int G, int fmt, uint16_t* y, void* ws,
                hipStream_t s) {
  if (fmt == 0) {
    if (G == 64) return launch_mt<0, 8>(c, x, M, K, N, packed, scale, zero, y, ws, s);
    return launch_mt<0, 16>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  }
  if (G == 64) return launch_mt<1, 8>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  return launch_mt<1, 16>(c, x, M, K, N, packed, scale, zero, y, ws, s);
}


}  // namespace w4

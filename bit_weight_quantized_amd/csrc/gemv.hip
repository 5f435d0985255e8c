// Decode-shaped W4 product y[M][N] = x[M][K] . W' for 1 <= M <= 32.
//
// The weight stream dominates: every packed byte is read once from HBM and
// turned into matrix-core operands on chip.  Dequantization is "after
// per-group mpGEMM" ("MixPE: Quantization and Hardware Co-design for Efficient
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
// Split K.  With S > 1 each workgroup leaves its fp32 partial in the workspace
// and the last one to finish a row block (a ticket counter) adds the S
// partials in slice order, writes y, and zeroes what it used, so results are
// deterministic and the workspace stays all-zero between calls.
#include "w4_device.h"
#include "w4_internal.h"

#include <cstdlib>

namespace w4 {
namespace {

constexpr int kGemvMaxThreads = 512;
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

// Shared-memory bytes of a workgroup: the staged activation slice, [8-position
// chunk of the slice][M] x 16 B (the same space later holds the cross-wave
// reduction).
__host__ __device__ inline int gemv_stage_bytes(int M, int slice_k) { return slice_k * 2 * M; }

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
// fp16 store, or with S > 1 the split-K partial and ticket protocol.
template <int MT>
__device__ __forceinline__ void gemv_finish(const f32x4 (&C)[MT], float* red, int* last_flag, int wave, int lane,
                                            int nwr, int nwk, int row_wg0, int M, int N, uint16_t* __restrict__ y,
                                            float* __restrict__ partial, uint32_t* __restrict__ tickets) {
  constexpr int kTile = MT * 256;
  const int S = gridDim.y;
  const int ks = blockIdx.y;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave * kTile + (t * 4 + i) * 64 + lane] = C[t][i];
  __syncthreads();

  // element e of the workgroup's output (nwr tiles of 16 rows x 16*MT tokens)
  auto coords = [&](int e, int& n, int& m, int& w_r, int& el) {
    w_r = e / kTile;
    el = e - w_r * kTile;
    const int l = el % 64;
    const int i = (el / 64) % 4;
    const int t = el / 256;
    n = row_wg0 + 16 * w_r + l % 16;
    m = t * 16 + 4 * (l / 16) + i;
  };
  auto wg_sum = [&](int w_r, int el) {
    float sum = 0.f;
    for (int k2 = 0; k2 < nwk; ++k2) sum += red[(k2 * nwr + w_r) * kTile + el];
    return sum;
  };

  const int total = nwr * kTile;
  if (S == 1) {
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
      int n, m, w_r, el;
      coords(e, n, m, w_r, el);
      if (m < M && n < N) y[(size_t)m * N + n] = float_to_half_bits(wg_sum(w_r, el));
    }
    return;
  }

  // ---- split-K: publish this slice's partial; the last arrival finishes.
  // Every access to the partials and tickets is an agent-scope atomic, which
  // this hardware performs at the device coherence point (write-through, not
  // left dirty in one XCD's L2).  Ordering comes from completion: each thread
  // waits until its partial stores are acknowledged, the barrier collects the
  // workgroup, and only then is the ticket incremented; the last arrival reads
  // the partials after observing the final ticket value.  This avoids the
  // whole-L2 write-back/invalidate an acquire-release fence costs per workgroup.
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    int n, m, w_r, el;
    coords(e, n, m, w_r, el);
    if (m < M && n < N)
      __hip_atomic_store(partial + ((size_t)ks * M + m) * N + n, wg_sum(w_r, el), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
  __builtin_amdgcn_s_waitcnt(0);  // all counters to zero: the stores above are acknowledged
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old =
        __hip_atomic_fetch_add(tickets + blockIdx.x, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *last_flag = (old == (uint32_t)(S - 1));
  }
  __syncthreads();
  if (!*last_flag) return;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    int n, m, w_r, el;
    coords(e, n, m, w_r, el);
    if (m < M && n < N) {
      float sum = 0.f;
      for (int k2 = 0; k2 < S; ++k2) {
        float* p = partial + ((size_t)k2 * M + m) * N + n;
        sum += __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // leave the workspace all-zero for the next call, whatever its shape
        __hip_atomic_store(p, 0.f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      y[(size_t)m * N + n] = float_to_half_bits(sum);
    }
  }
  if (threadIdx.x == 0) __hip_atomic_store(tickets + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int LB, int MT, int R>
__global__ __launch_bounds__(kGemvMaxThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    float* __restrict__ partial, uint32_t* __restrict__ tickets, int nwr, int nwk) {
  constexpr int G = 8 * LB;
  constexpr int GPT = kTileK / G;  // groups per tile: 1 (G=128) or 2 (G=64)
  constexpr int WPG = 4 / GPT;     // 4-byte words (one product each) per group
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];
  __shared__ int last_flag;

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

  // tile ranges: the workgroup's slice [ts0, ts1), the wave's run [t0, t0 + cnt)
  const int ts0 = (int)((long)KT * ks / S), ts1 = (int)((long)KT * (ks + 1) / S);
  const int t0 = ts0 + (int)((long)(ts1 - ts0) * wk / nwk);
  const int cnt = ts0 + (int)((long)(ts1 - ts0) * (wk + 1) / nwk) - t0;
  const int t_last = t0 + max(cnt, 1) - 1;
  const int k0 = ts0 * kTileK;  // first K position of the slice
  // this wave's tile column; a wave past the last one (only in a partial last
  // row block) re-reads the last column and stores nothing
  const int colw = min(row_wg0 / 16 + wr, N / 16 - 1);

  u32x4* xs = reinterpret_cast<u32x4*>(smem);

  // Staging.  One unit = 8 consecutive activations of token row m (chunk r of
  // the slice: K positions k0 + 8 r .. + 7), r fastest so loads coalesce; it is
  // the A operand of lane (kb = r % 4, m) for word (r / 4) % 4 of tile r / 16.
  const int n_chunks = (ts1 - ts0) * (kTileK / 8);
  const int n_xu = n_chunks * M;
  const float inv_nc = 1.0f / (float)n_chunks;
  auto load_xunit = [&](int u) {
    int m, r;
    div_small(u, n_chunks, inv_nc, m, r);
    return *reinterpret_cast<const u32x4*>(x + (size_t)m * K + k0 + 8 * r);
  };
  auto store_xunit = [&](u32x4 q, int u) {
    int m, r;
    div_small(u, n_chunks, inv_nc, m, r);
    if constexpr (FMT == 0) {
      // (x0,x1), (x2,x3)/16, (x4,x5), (x6,x7)/16: the order and scale the INT4 masks produce
      q = u32x4{q.x, pk_mul_f16(q.y, kHalfSixteenthPair), q.z, pk_mul_f16(q.w, kHalfSixteenthPair)};
    } else {
      // (x0,x2), (x4,x6), (x1,x3), (x5,x7): the level pairs of bytes 0..3 of a word
      q = u32x4{pair_lo(q.x, q.y), pair_lo(q.z, q.w), pair_hi(q.x, q.y), pair_hi(q.z, q.w)};
    }
    xs[r * M + m] = q;
  };

  // Ring slot: the lane's 16 bytes of a weight tile and the tile's scale and
  // zero point for the lane's row (G = 64: both groups, low half first).
  struct Slot {
    u32x4 w;
    uint32_t s, z;
  };
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, (uint32_t)((size_t)N * (K / 2)));
  const uint32_t voff = (uint32_t)lane * 16;
  const uint32_t col_base = (uint32_t)colw * (uint32_t)KT;
  const size_t srow = (size_t)(colw * 16 + ln) * ng;
  auto load_slot = [&](Slot& sl, int t) {
    // a wave without tiles (more waves than tiles) still loads: keep it in bounds
    const int tt = __builtin_amdgcn_readfirstlane(min(min(t, t_last), KT - 1));
    sl.w = buffer_load16(wrs, voff, (col_base + (uint32_t)tt) * (uint32_t)kTileBytes);
    if constexpr (GPT == 1) {
      sl.s = scale[srow + tt];
      sl.z = FMT == 0 ? (uint32_t)zero[srow + tt] : 0u;
    } else {
      sl.s = *reinterpret_cast<const uint32_t*>(scale + srow + 2 * tt);
      sl.z = FMT == 0 ? *reinterpret_cast<const uint32_t*>(zero + srow + 2 * tt) : 0u;
    }
  };

  // ---- 1. first staging batch (clamped index: every thread loads), then the
  // weight ring, so the staging loads are the older ones and never wait
  // behind weight traffic
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  constexpr int kXB = 4;  // x units per thread per batch
  u32x4 xb[kXB];
#pragma unroll
  for (int i = 0; i < kXB; ++i) xb[i] = load_xunit(min(tid + i * nthr, n_xu - 1));
  Slot ring[R];
#pragma unroll
  for (int d = 0; d < R; ++d) load_slot(ring[d], t0 + d);

  // ---- 2. finish staging
  for (int base = 0; base < n_xu; base += kXB * nthr) {
    if (base > 0) {
#pragma unroll
      for (int i = 0; i < kXB; ++i) xb[i] = load_xunit(min(base + tid + i * nthr, n_xu - 1));
    }
#pragma unroll
    for (int i = 0; i < kXB; ++i) {
      const int u = base + tid + i * nthr;
      if (u < n_xu) store_xunit(xb[i], u);
    }
  }
  if constexpr (FMT == 1) {
    for (int i = tid; i < 256; i += nthr)
      lut[i] = (uint32_t)float_to_half_bits(nf4_level(i & 15)) |
               ((uint32_t)float_to_half_bits(nf4_level(i >> 4)) << 16);
  }
  __syncthreads();

  f32x4 C[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) C[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  int mrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) mrow[t] = min(t * 16 + ln, M - 1);
  // INT4: the group's activation sum per token, as a product with constant B
  // (1 for the even pairs, 16 for the pre-scaled odd pairs)
  const u32x4 kSumB{0x3C003C00u, 0x4C004C00u, 0x3C003C00u, 0x4C004C00u};

  // products of one tile (tl: tile index within the slice), group by group
  auto compute_tile = [&](const Slot& sl, int tl) {
    u32x4 B[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t a = sl.w[w];
      if constexpr (FMT == 0) {
        const uint32_t as = a >> 8;
        B[w] = u32x4{a & 0x000F000Fu, a & 0x00F000F0u, as & 0x000F000Fu, as & 0x00F000F0u};
      } else {
        B[w] = u32x4{lut[a & 0xFFu], lut[(a >> 8) & 0xFFu], lut[(a >> 16) & 0xFFu], lut[a >> 24]};
      }
    }
    const u32x4* xa = xs + (size_t)(tl * 16 + kb) * M;  // + (4 w) * M + m
#pragma unroll
    for (int gi = 0; gi < GPT; ++gi) {
      const float sv = half_bits_to_float((uint16_t)(sl.s >> (16 * gi)));
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = gi * WPG; w < (gi + 1) * WPG; ++w) acc = mfma_f16(xa[(4 * w) * M + mrow[t]], B[w], acc);
        if constexpr (FMT == 0) {
          f32x4 sx = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int w = gi * WPG; w < (gi + 1) * WPG; ++w) sx = mfma_f16(xa[(4 * w) * M + mrow[t]], kSumB, sx);
          const float zv = half_bits_to_float((uint16_t)(sl.z >> (16 * gi)));
          const float ex = sv * 16777216.0f, ey = -sv * zv;  // codes enter as q * 2^-24
#pragma unroll
          for (int i = 0; i < 4; ++i) C[t][i] = fmaf(ex, acc[i], fmaf(ey, sx[i], C[t][i]));
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) C[t][i] = fmaf(sv, acc[i], C[t][i]);
        }
      }
    }
  };

  if (cnt > 0) {
    const int cnt_pad = (cnt + R - 1) / R * R;
    int base = 0;
    // steady state: every block of R tiles but the last refills the ring.
    // A slot is consumed before its refill is issued, so the refill lands in
    // the same registers: moving a register whose load is still in flight
    // would make the wave wait for it (draining the ring every R tiles).
    for (; base + R < cnt_pad; base += R) {
#pragma unroll
      for (int d = 0; d < R; ++d) {
        const int ci = base + d;
        if (ci < cnt) compute_tile(ring[d], t0 + ci - ts0);
        load_slot(ring[d], t0 + ci + R);
      }
    }
    // last block: no refill
#pragma unroll
    for (int d = 0; d < R; ++d) {
      const int ci = base + d;
      if (ci < cnt) compute_tile(ring[d], t0 + ci - ts0);
    }
  }

  // ---- cross-wave reduction (over wk) through LDS, reusing the staging area
  __syncthreads();
  gemv_finish<MT>(C, reinterpret_cast<float*>(smem), &last_flag, wave, lane, nwr, nwk, row_wg0, M, N, y, partial,
                  tickets);
}

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

constexpr int kGemvLdsTarget = 76 * 1024;  // two workgroups per CU

}  // namespace

GemvPlan plan_gemv(int M, int K, int N, int G) {
  GemvPlan c;
  const int KT = K / kTileK;  // tiles per 16-row column
  c.mt = M <= 16 ? 1 : 2;
  c.ring = 4;
  // Measured on MI355X (K = N = 8192, M = 1..16, both formats): one 16-row
  // tile column per workgroup for M <= 2, two beyond (the staged activations
  // then serve twice the weight rows); four K waves per workgroup; K split
  // over workgroups until the grid holds about 2048 waves.
  c.nwr = M <= 2 ? 1 : 2;
  c.nwk = 4;
  const int want_waves = 2048;
  c.row_blocks = (N + 16 * c.nwr - 1) / (16 * c.nwr);
  c.s = 1;
  while (c.row_blocks * c.s * c.nwr * c.nwk < want_waves && KT / (c.s * 2 * c.nwk) >= 8) c.s *= 2;
  // long rows: more K waves (up to 8) keep at most about 32 tiles per wave
  while (c.nwk < 8 && c.nwr * c.nwk * 2 <= kGemvMaxThreads / kWave && KT / (c.s * c.nwk) > 32) c.nwk *= 2;
  const int ring = env_int("W4_GEMV_RING", 0);
  const int nwr = env_int("W4_GEMV_NWR", 0);
  const int nwk = env_int("W4_GEMV_NWK", 0);
  const int s = env_int("W4_GEMV_S", 0);
  if (ring == 4 || ring == 8) c.ring = ring;
  if (nwr >= 1 && nwr <= 8) c.nwr = nwr;
  if (nwk >= 1 && nwk <= 8) c.nwk = nwk;
  if (s >= 1 && s <= KT) c.s = s;
  if (c.nwr * c.nwk > kGemvMaxThreads / kWave) c.nwk = kGemvMaxThreads / kWave / c.nwr;
  // shrink the activation slice (more K splits) until the workgroup fits in LDS
  for (;;) {
    const int slice_tiles = (KT + c.s - 1) / c.s;
    const int stage = gemv_stage_bytes(M, slice_tiles * kTileK);
    const int red = c.nwr * c.nwk * c.mt * 256 * 4;
    c.lds_bytes = (size_t)(stage > red ? stage : red);
    if ((int)c.lds_bytes <= kGemvLdsTarget || c.s >= KT) break;
    ++c.s;
  }
  c.row_blocks = (N + 16 * c.nwr - 1) / (16 * c.nwr);
  c.ws_partial_bytes = c.s > 1 ? ((size_t)c.s * M * N * sizeof(float) + 255) / 256 * 256 : 0;
  c.ws_bytes = c.s > 1 ? c.ws_partial_bytes + (size_t)c.row_blocks * sizeof(uint32_t) : 0;
  return c;
}

namespace {

template <int FMT, int LB, int MT>
int launch_t(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
             const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  const dim3 block(c.nwr * c.nwk * kWave);
  const dim3 grid((unsigned)c.row_blocks, (unsigned)c.s);
  float* partial = c.s > 1 ? static_cast<float*>(ws) : nullptr;
  uint32_t* tickets =
      c.s > 1 ? reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + c.ws_partial_bytes) : nullptr;
  if (c.ring == 4)
    hipLaunchKernelGGL((gemv_kernel<FMT, LB, MT, 4>), grid, block, c.lds_bytes, s, x, M, K, N, packed, scale, zero,
                       y, partial, tickets, c.nwr, c.nwk);
  else
    hipLaunchKernelGGL((gemv_kernel<FMT, LB, MT, 8>), grid, block, c.lds_bytes, s, x, M, K, N, packed, scale, zero,
                       y, partial, tickets, c.nwr, c.nwk);
  return check_launch("gemv");
}

template <int FMT, int LB>
int launch_mt(const GemvPlan& c, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
              const uint16_t* scale, const uint16_t* zero, uint16_t* y, void* ws, hipStream_t s) {
  if (c.mt == 1) return launch_t<FMT, LB, 1>(c, x, M, K, N, packed, scale, zero, y, ws, s);
  return launch_t<FMT, LB, 2>(c, x, M, K, N, packed, scale, zero, y, ws, s);
}

}  // namespace

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

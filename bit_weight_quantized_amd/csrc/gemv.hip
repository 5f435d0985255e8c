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
// Work split.  Grid = (row blocks of 16*NWR weight rows) x (S slices of K).  A
// workgroup has NWR x NWK waves: wave (wr, wk) owns 16 rows and a contiguous
// run of 256-byte column chunks of its slice.  The workgroup first stages in
// LDS, once, everything its waves share: the activation slice, already laid
// out as matrix-core A operands, and the rows' scales and zero points.
//
// Weight stream.  A wave reads its rows in chunks of 16 rows x 256 bytes: each
// load instruction covers 4 rows x 256 contiguous bytes, the shape that reaches
// the streaming-read bandwidth (narrower per-row runs lose about a third on
// MI355X).  Chunks are prefetched D deep into a register ring, so the
// vector-memory counter only waits on the oldest chunk; everything else comes
// from LDS on its own counter.  Each chunk is written to a per-wave 4 KB LDS
// tile with an XOR swizzle (16-byte slot s of row r lands in slot s ^ r), which
// makes both that write and the matrix-core-layout reads bank-conflict free.
//
// Matrix-core mapping (v_mfma_f32_16x16x32_f16): weight rows are the MFMA "n"
// dimension, tokens the "m" dimension.  Lane l serves row l%16 and k-block
// kb = l/16; per group it takes LB packed bytes (2*LB codes) at
// k = g*G + kb*2*LB, with G = 8*LB, so a group never splits an MFMA.  Token rows
// past M read row M-1 and weight rows past N read row N-1 (valid addresses,
// never stored), which keeps every load unconditional.
//
// INT4 operands.  A code q in the low nibble of an fp16 lane is the subnormal
// value q * 2^-24 exactly, and in bits 4..7 it is q * 2^-20; masking the packed
// word therefore yields exact fp16 operands in 5 VALU ops per 8 codes, with no
// offset to cancel.  Odd-position codes (2^-20) meet activations pre-scaled by
// 1/16, so every product is x*q*2^-24.  The zero point is applied with the
// group's activation sum: y += s * (2^24 * sum x*q - z * sum x), where the sum
// comes from the same A operands times a constant B on the matrix cores.
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
constexpr int kChunkBytes = 256;  // per-row span of one chunk

// fp16 pair constants
constexpr uint32_t kHalfOnePair = 0x3C003C00u;        // (1.0, 1.0)
constexpr uint32_t kHalfSixteenPair = 0x4C004C00u;    // (16.0, 16.0)
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

// Shared-memory layout of a workgroup (dynamic LDS), byte offsets.
struct GemvLds {
  int xs;    // A operands: [slice group][kb][NV][M] x 16 B
  int sxp;   // INT4 partial activation sums: [slice group][kb][M] floats
  int sx;    // INT4 activation sums: [slice group][16*MT] floats
  int ep;    // epilogue factors per (slice group, row): INT4 (s*2^24, -s*z), NF4 (s, 0)
  int tile;  // per-wave transpose tiles: [waves][16 rows][256 B]
  int total;
};

__host__ __device__ inline int align16(int v) { return (v + 15) & ~15; }

__host__ __device__ inline GemvLds gemv_lds_layout(int M, int MT, int G, int slice_groups, int rows, int waves) {
  GemvLds L;
  L.xs = 0;
  L.sxp = align16(L.xs + slice_groups * G * 2 * M);
  L.sx = align16(L.sxp + slice_groups * 4 * M * 4);
  L.ep = align16(L.sx + slice_groups * 16 * MT * 4);
  L.tile = align16(L.ep + slice_groups * rows * 8);
  L.total = L.tile + waves * 16 * kChunkBytes;
  return L;
}

template <int FMT, int LB, int MT, int kRing>
__global__ __launch_bounds__(kGemvMaxThreads) void gemv_kernel(
    const uint16_t* __restrict__ x, int M, int K, int N, const uint8_t* __restrict__ packed,
    const uint16_t* __restrict__ scale, const uint16_t* __restrict__ zero, uint16_t* __restrict__ y,
    float* __restrict__ partial, uint32_t* __restrict__ tickets, int nwr, int nwk) {
  constexpr int G = 8 * LB;
  constexpr int CG = kChunkBytes / (G / 2);  // groups per chunk: 4 (G=128) or 8 (G=64)
  constexpr int NV = LB / 4;                 // 16-byte A-operand pieces per lane per group
  constexpr int NP = NV / 2;                 // INT4: (even, odd) MFMA pairs per group
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t lut[FMT == 1 ? 256 : 1];
  __shared__ int last_flag;

  const int lane = threadIdx.x % kWave;
  // wave-uniform by construction; readfirstlane lets the compiler keep it (and
  // everything derived from it) in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int nw = nwr * nwk;
  const int wr = wave % nwr;
  const int wk = wave / nwr;
  const int ln = lane % 16;
  const int kb = lane / 16;
  const int ng = K / G;
  const int rows_wg = 16 * nwr;
  const int row_wg0 = blockIdx.x * rows_wg;
  const int row0 = row_wg0 + 16 * wr;  // this wave's 16 rows
  const int S = gridDim.y;
  const int ks = blockIdx.y;
  const int row_bytes = K / 2;

  // chunk ranges: the workgroup's slice [cs0, cs1), the wave's run [c0, c0 + cnt)
  const int CT = (row_bytes + kChunkBytes - 1) / kChunkBytes;
  const int cs0 = (int)((long)CT * ks / S), cs1 = (int)((long)CT * (ks + 1) / S);
  const int c0 = cs0 + (int)((long)(cs1 - cs0) * wk / nwk);
  const int cnt = cs0 + (int)((long)(cs1 - cs0) * (wk + 1) / nwk) - c0;
  const int c_last = c0 + cnt - 1;
  const int gs0 = cs0 * CG;
  const int gs1 = min(cs1 * CG, ng);
  const int SG = gs1 - gs0;  // groups in the slice

  const GemvLds L = gemv_lds_layout(M, MT, G, max(cs1 - cs0, 1) * CG, rows_wg, nw);
  u32x4* xs = reinterpret_cast<u32x4*>(smem + L.xs);
  float* sxp = reinterpret_cast<float*>(smem + L.sxp);
  float* sxs = reinterpret_cast<float*>(smem + L.sx);
  float2* eps = reinterpret_cast<float2*>(smem + L.ep);
  unsigned char* tile = smem + L.tile + wave * 16 * kChunkBytes;

  // Staging units.  x: one unit = one (group, k-block) of one token row, i.e.
  // 2*LB activations (4*LB bytes), m fastest so consecutive threads write
  // consecutive LDS words.  Scales/zeros: one unit = 4 consecutive groups of
  // one row.  Each thread's first unit of each kind is loaded before the
  // weight ring (older loads), so staging never waits behind weight traffic;
  // further units (large M or long slices) are staged after the ring.
  const int n_xu = SG * 4 * M;
  const int sg4 = (SG + 3) / 4;
  const int n_su = rows_wg * sg4;
  struct XUnit { u32x4 q[NV]; };
  auto xunit_src = [&](int u) {
    const int m = u % M;
    const int r = u / M;  // = gl * 4 + b
    return x + (size_t)m * K + (size_t)gs0 * G + (size_t)r * 2 * LB;
  };
  auto load_xunit = [&](XUnit& xu, int u) {
    const u32x4* src = reinterpret_cast<const u32x4*>(xunit_src(u));
#pragma unroll
    for (int v = 0; v < NV; ++v) xu.q[v] = src[v];
  };
  auto store_xunit = [&](const XUnit& xu, int u) {
    const int m = u % M;
    const int r = u / M;
    u32x4* dst = xs + (size_t)r * NV * M + m;
    if constexpr (FMT == 0) {
      float ssum = 0.f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t X[8] = {xu.q[2 * p].x, xu.q[2 * p].y, xu.q[2 * p].z, xu.q[2 * p].w,
                               xu.q[2 * p + 1].x, xu.q[2 * p + 1].y, xu.q[2 * p + 1].z, xu.q[2 * p + 1].w};
        const u32x4 ae{pair_lo(X[0], X[2]), pair_lo(X[1], X[3]), pair_lo(X[4], X[6]), pair_lo(X[5], X[7])};
        const u32x4 ao{pk_mul_f16(pair_hi(X[0], X[2]), kHalfSixteenthPair),
                       pk_mul_f16(pair_hi(X[1], X[3]), kHalfSixteenthPair),
                       pk_mul_f16(pair_hi(X[4], X[6]), kHalfSixteenthPair),
                       pk_mul_f16(pair_hi(X[5], X[7]), kHalfSixteenthPair)};
        dst[(2 * p) * M] = ae;
        dst[(2 * p + 1) * M] = ao;
        // the activations exactly as the matrix cores see them (odd ones as 16 * fp16(x/16))
#pragma unroll
        for (int i = 0; i < 4; ++i) ssum += lo_half(ae[i]) + hi_half(ae[i]) + 16.0f * (lo_half(ao[i]) + hi_half(ao[i]));
      }
      sxp[u] = ssum;  // [gl][kb][m] == unit index
    } else {
#pragma unroll
      for (int v = 0; v < NV; ++v) dst[v * M] = xu.q[v];
    }
  };
  struct SUnit { uint16_t s[4], z[4]; };
  auto load_sunit = [&](SUnit& su, int u) {
    const int r = u / sg4;
    const int g4 = (u - r * sg4) * 4;
    const size_t rowoff = (size_t)min(row_wg0 + r, N - 1) * ng + gs0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const size_t o = rowoff + min(g4 + i, SG - 1);
      su.s[i] = scale[o];
      if constexpr (FMT == 0) su.z[i] = zero[o];
    }
  };
  auto store_sunit = [&](const SUnit& su, int u) {
    const int r = u / sg4;
    const int g4 = (u - r * sg4) * 4;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (g4 + i < SG) {
        const float sv = half_bits_to_float(su.s[i]);
        float2 e;
        if constexpr (FMT == 0) {
          e.x = sv * 16777216.0f;  // the codes enter the products as q * 2^-24
          e.y = -sv * half_bits_to_float(su.z[i]);
        } else {
          e.x = sv;
          e.y = 0.f;
        }
        eps[(g4 + i) * rows_wg + r] = e;
      }
  };

  // ---- 1. first staging unit of each kind (clamped index: every thread loads)
  XUnit xu0;
  SUnit su0;
  const int tid = threadIdx.x;
  load_xunit(xu0, min(tid, n_xu - 1));
  load_sunit(su0, min(tid, n_su - 1));

  // ---- 2. weight ring prologue
  // Load role of a lane: row 4*i + lane/16 of the wave's 16 rows, 16-byte slot
  // lane%16 of the chunk.  Buffer addressing: a constant per-lane offset plus
  // the chunk base in a scalar register; rows past N and bytes past a short
  // last chunk read zeros or neighbouring bytes that are never used.
  const int lrow = lane / 16;
  const int lslot = lane % 16;
  const __amdgpu_buffer_rsrc_t wrs = make_rsrc(packed, (uint32_t)((size_t)N * row_bytes));
  uint32_t voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) voff[i] = (uint32_t)(row0 + 4 * i + lrow) * (uint32_t)row_bytes + lslot * 16;
  u32x4 ring[kRing][4];
  if (cnt > 0) {
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      const uint32_t soff = (uint32_t)min(c0 + d, c_last) * kChunkBytes;
#pragma unroll
      for (int i = 0; i < 4; ++i) ring[d][i] = buffer_load16(wrs, voff[i], soff);
    }
  }

  // ---- 3. finish staging: first units, then any remaining ones
  if (tid < n_xu) store_xunit(xu0, tid);
  if (tid < n_su) store_sunit(su0, tid);
  for (int u = tid + blockDim.x; u < n_xu; u += blockDim.x) {
    XUnit xu;
    load_xunit(xu, u);
    store_xunit(xu, u);
  }
  for (int u = tid + blockDim.x; u < n_su; u += blockDim.x) {
    SUnit su;
    load_sunit(su, u);
    store_sunit(su, u);
  }
  if constexpr (FMT == 1) {
    for (int b = tid; b < 256; b += blockDim.x)
      lut[b] = (uint32_t)float_to_half_bits(nf4_level(b & 15)) |
               ((uint32_t)float_to_half_bits(nf4_level(b >> 4)) << 16);
  }
  __syncthreads();
  if constexpr (FMT == 0) {
    // per-group activation sums from the per-unit partials (fixed order)
    for (int t = tid; t < SG * 16 * MT; t += blockDim.x) {
      const int gl = t / (16 * MT);
      const int m = t - gl * 16 * MT;
      float v = 0.f;
      if (m < M) {
#pragma unroll
        for (int b = 0; b < 4; ++b) v += sxp[(gl * 4 + b) * M + m];
      }
      sxs[t] = v;
    }
    __syncthreads();
  }

  f32x4 C[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) C[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  int mrow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) mrow[t] = min(t * 16 + ln, M - 1);

  // chunk -> the wave's LDS tile (swizzled), then its CG groups from the tile
  auto write_tile = [&](const u32x4 (&w)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * i + lrow;
      *reinterpret_cast<u32x4*>(tile + r * kChunkBytes + ((lslot ^ r) << 4)) = w[i];
    }
  };
  const int rloc = 16 * wr + ln;
  // operands of one group gathered from LDS, then its products
  struct GOps {
    uint32_t bw[NV];
    float2 e;
  };
  auto gather = [&](GOps& o, int j, int gl) {
    const int byte = j * (G / 2) + kb * LB;
    const unsigned char* src = tile + ln * kChunkBytes + (((byte >> 4) ^ ln) << 4) + (byte & 15);
    if constexpr (LB == 16) {
      const u32x4 q = *reinterpret_cast<const u32x4*>(src);
      o.bw[0] = q.x;
      o.bw[1] = q.y;
      o.bw[2] = q.z;
      o.bw[3] = q.w;
    } else {
      const u32x2 q = *reinterpret_cast<const u32x2*>(src);
      o.bw[0] = q.x;
      o.bw[1] = q.y;
    }
    o.e = eps[gl * rows_wg + rloc];
  };
  auto math = [&](const GOps& o, int gl, float live) {
    const u32x4* xa = xs + ((size_t)(gl * 4 + kb) * NV) * M;
    if constexpr (FMT == 0) {
      u32x4 BE[NP], BO[NP];
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const uint32_t v0 = o.bw[2 * p], v1 = o.bw[2 * p + 1];
        const uint32_t v0s = v0 >> 8, v1s = v1 >> 8;
        BE[p] = u32x4{v0 & 0x000F000Fu, v0s & 0x000F000Fu, v1 & 0x000F000Fu, v1s & 0x000F000Fu};
        BO[p] = u32x4{v0 & 0x00F000F0u, v0s & 0x00F000F0u, v1 & 0x00F000F0u, v1s & 0x00F000F0u};
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          acc = mfma_f16(xa[(2 * p) * M + mrow[t]], BE[p], acc);
          acc = mfma_f16(xa[(2 * p + 1) * M + mrow[t]], BO[p], acc);
        }
        const f32x4 sx = *reinterpret_cast<const f32x4*>(sxs + gl * 16 * MT + t * 16 + 4 * kb);
        const float a = o.e.x * live, b = o.e.y * live;
#pragma unroll
        for (int i = 0; i < 4; ++i) C[t][i] = fmaf(a, acc[i], fmaf(b, sx[i], C[t][i]));
      }
    } else {
      u32x4 B[NV];
#pragma unroll
      for (int u = 0; u < NV; ++u) {
        const uint32_t v = o.bw[u];
        B[u] = u32x4{lut[v & 0xFFu], lut[(v >> 8) & 0xFFu], lut[(v >> 16) & 0xFFu], lut[v >> 24]};
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NV; ++u) acc = mfma_f16(xa[u * M + mrow[t]], B[u], acc);
        const float a = o.e.x * live;
#pragma unroll
        for (int i = 0; i < 4; ++i) C[t][i] = fmaf(a, acc[i], C[t][i]);
      }
    }
  };
  auto compute_tile = [&](int c) {
    const int jn = min(CG, gs1 - c * CG);  // groups of this chunk (the last chunk of a row may be short)
    const int gl0 = c * CG - gs0;
    if (jn == CG) {
      // full chunk: fully unrolled, two groups in flight at a time
#pragma unroll
      for (int j = 0; j < CG; j += 2) {
        GOps o0, o1;
        gather(o0, j, gl0 + j);
        gather(o1, j + 1, gl0 + j + 1);
        math(o0, gl0 + j, 1.0f);
        math(o1, gl0 + j + 1, 1.0f);
      }
    } else {
#pragma unroll 1
      for (int j = 0; j < jn; ++j) {
        GOps o0;
        gather(o0, j, gl0 + j);
        math(o0, gl0 + j, 1.0f);
      }
    }
  };

  if (cnt > 0) {
    const int cnt_pad = (cnt + kRing - 1) / kRing * kRing;
    int base = 0;
    // steady state: every block of kRing chunks but the last refills the ring
    for (; base + kRing < cnt_pad; base += kRing) {
#pragma unroll
      for (int d = 0; d < kRing; ++d) {
        const int ci = base + d;
        write_tile(ring[d]);
        const uint32_t soff = (uint32_t)min(c0 + ci + kRing, c_last) * kChunkBytes;
#pragma unroll
        for (int i = 0; i < 4; ++i) ring[d][i] = buffer_load16(wrs, voff[i], soff);
        if (ci < cnt) compute_tile(c0 + ci);
      }
    }
    // last block: no refill
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      const int ci = base + d;
      if (ci < cnt) {
        write_tile(ring[d]);
        compute_tile(c0 + ci);
      }
    }
  }

  // ---- cross-wave reduction (over wk) through LDS, reusing the staging area
  constexpr int kTile = MT * 256;
  float* red = reinterpret_cast<float*>(smem);
  __syncthreads();
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
    last_flag = (old == (uint32_t)(S - 1));
  }
  __syncthreads();
  if (!last_flag) return;
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

int env_int(const char* name, int dflt) {
  const char* v = std::getenv(name);
  if (!v || !*v) return dflt;
  return std::atoi(v);
}

constexpr int kGemvLdsTarget = 76 * 1024;  // two workgroups per CU

}  // namespace

GemvPlan plan_gemv(int M, int K, int N, int G) {
  GemvPlan c;
  const int cg = kChunkBytes / (G / 2);
  const int CT = (K / 2 + kChunkBytes - 1) / kChunkBytes;  // chunks per row
  c.mt = M <= 16 ? 1 : 2;
  c.ring = 2;
  // Rows per workgroup grow with M so the staged activations serve more
  // weight rows; K is split over workgroups until the grid covers the GPU
  // (measured on MI355X for the 8192 x 8192 and 8192 x 28672 layers).
  c.nwr = M <= 2 ? 1 : 2;
  c.nwk = M <= 8 ? 4 : 2;
  const int want_wgs = M <= 8 ? 512 : 1024;
  c.row_blocks = (N + 16 * c.nwr - 1) / (16 * c.nwr);
  c.s = 1;
  while (c.row_blocks * c.s < want_wgs && c.s * 2 * c.nwk <= CT) c.s *= 2;
  // long rows: more K waves (up to 8) keep about 4 chunks per wave
  while (c.nwk < 8 && CT / (c.s * c.nwk) > 8) c.nwk *= 2;
  const int ring = env_int("W4_GEMV_RING", 0);
  const int nwr = env_int("W4_GEMV_NWR", 0);
  const int nwk = env_int("W4_GEMV_NWK", 0);
  const int s = env_int("W4_GEMV_S", 0);
  if (ring == 2 || ring == 4) c.ring = ring;
  if (nwr >= 1 && nwr <= 8) c.nwr = nwr;
  if (nwk >= 1 && nwk <= 8) c.nwk = nwk;
  if (s >= 1 && s <= CT) c.s = s;
  if (c.nwr * c.nwk > kGemvMaxThreads / kWave) c.nwk = kGemvMaxThreads / kWave / c.nwr;
  // shrink the activation slice (more K splits) until the workgroup fits in LDS
  for (;;) {
    const int slice_chunks = (CT + c.s - 1) / c.s;
    const GemvLds L = gemv_lds_layout(M, c.mt, G, slice_chunks * cg, 16 * c.nwr, c.nwr * c.nwk);
    const int red = c.nwr * c.nwk * c.mt * 256 * 4;
    c.lds_bytes = (size_t)(L.total > red ? L.total : red);
    if ((int)c.lds_bytes <= kGemvLdsTarget || c.s >= CT) break;
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
  if (c.ring == 2)
    hipLaunchKernelGGL((gemv_kernel<FMT, LB, MT, 2>), grid, block, c.lds_bytes, s, x, M, K, N, packed, scale, zero,
                       y, partial, tickets, c.nwr, c.nwk);
  else
    hipLaunchKernelGGL((gemv_kernel<FMT, LB, MT, 4>), grid, block, c.lds_bytes, s, x, M, K, N, packed, scale, zero,
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

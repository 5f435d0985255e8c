/*
 * w4.h -- C ABI of a 4-bit weight-quantized matmul library for AMD MI355X
 * (gfx950, CDNA4).
 *
 * The library computes y = x . W' where x is fp16 activations [M][K] and W' is
 * a 4-bit quantized weight matrix, either INT4 with a per-group scale and zero
 * point or NF4 (16-level NormalFloat codebook) with a per-block absmax.  This
 * is the mixed-precision GEMM (low-precision weights times higher-precision
 * activations) of the page "MixPE: Quantization and Hardware Co-design for
 * Efficient LLM Inference" (Abstract).
 *
 * Pages cited below by short name (title, section):
 *   [MSD]   "Multi-Scale Dequant: Eliminating Dequantization Bottleneck via
 *           Activation Decomposition for Efficient LLM Inference", Abstract.
 *   [MixPE] "MixPE: Quantization and Hardware Co-design for Efficient LLM
 *           Inference", Abstract.
 *   [NF4]   "Fast NF4 Dequantization Kernels for Large Language Model
 *           Inference", Abstract.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layouts.  The weight is stored transposed, W^T [N][K], K contiguous (the
 *   PyTorch Linear weight layout).  Codes are one byte each, [N][K].  Packed
 *   weights (this library's own encoding, N*K/2 bytes) are a sequence of
 *   1024-byte tiles, each holding 16 weight rows x 128 K positions; tile
 *   (nb, kb) covers rows 16nb..16nb+15 and K positions 128kb..128kb+127 and
 *   sits at byte offset (nb * K/128 + kb) * 1024.  Within a tile, the 16
 *   bytes at offset 16*(16j + r) hold row r (0..15), j = 0..3, as four
 *   little-endian 32-bit words; word t (0..3) holds the codes of K positions
 *   32t + 8j + e, e = 0..7, with offset e in nibble p where e = (0, 2, 4, 6,
 *   1, 3, 5, 7)[p] (nibble p = bits 4p..4p+3).  This puts one 64-lane
 *   wavefront's 16-byte loads on one contiguous kilobyte and lets the
 *   masks 0x000F000F << 4i pick out the adjacent code pairs (8j+2i, 8j+2i+1).
 *   Per-group scales, zero points and NF4 absmax values are fp16 [N][K/G]
 *   (group g covers k in [g*G, (g+1)*G)).  Zero points are integers 0..15
 *   stored as fp16.  Activations x are fp16 [M][K]; outputs y are fp16
 *   [M][N]; all row-major.  fp16 values travel as uint16_t bit patterns.
 * Memory.  Every pointer argument except those marked "host" is a device
 *   pointer on the current HIP device.  The caller owns every buffer; the
 *   library allocates nothing and keeps no state besides a thread-local
 *   error string.  Device pointers must be 16-byte aligned.
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *   stream).  Calls only enqueue work and never synchronize; outputs are valid
 *   once the stream reaches that point.  Calls that share a workspace must be
 *   ordered on one stream.
 * Errors.  Arguments are checked before anything is enqueued.  A failed check
 *   returns a negative w4_status and enqueues nothing; w4_last_error() then
 *   describes the failure.  A launch failure reported by HIP returns W4_EHIP.
 *   No C++ exception crosses this boundary.
 * Shape rules.  G (group or block size along K) is 64 or 128; K % G == 0;
 *   entry points that take packed weights also need K % 128 == 0 and
 *   N % 16 == 0 (whole tiles) and N * K / 2 < 4 GiB; M >= 1.  NF4 takes
 *   zero == NULL; INT4 needs zero != NULL.
 */
#ifndef W4_H_
#define W4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  W4_OK = 0,
  W4_EINVAL = -1,        /* bad shape, null or misaligned pointer, bad enum */
  W4_EUNSUPPORTED = -2,  /* valid request this entry point does not serve */
  W4_EWORKSPACE = -3,    /* workspace missing or smaller than required */
  W4_EHIP = -4           /* the HIP runtime reported an error */
} w4_status;

typedef enum { W4_INT4_ASYM = 0, W4_NF4 = 1 } w4_fmt;

/* W4_DQ_F16: weights are dequantized to fp16 (s*(q-z), or c[idx]*a) before
 *   the fp16 matrix-core product (the dequantization baseline of [MSD], [NF4]).
 * W4_POSTSCALE: the integer codes (q-z), or the NF4 levels c[idx], enter the
 *   fp16 product unscaled; each group's fp32 partial sum is multiplied by its
 *   scale after accumulation ([MixPE]: the dequantization moves after the
 *   per-group product). */
typedef enum { W4_DQ_F16 = 0, W4_POSTSCALE = 1 } w4_mode;

typedef enum {
  W4_OP_QUANTIZE = 0,
  W4_OP_PACK = 1,
  W4_OP_GEMV = 2,
  W4_OP_GEMM = 3,
  W4_OP_GEMM_DECOMP = 4,
  W4_OP_GEMM_MX = 5,
  W4_OP_ATTN_MSD = 6,
  W4_OP_GEMM_DECOMP_FUSED = 7
} w4_op;

/*
 * w4_quantize -- quantize fp32 weights W^T [N][K] per group of G along K.
 *
 * fmt == W4_INT4_ASYM ([MixPE]: one scale and one zero point per group), per
 * group, in fp64: lo = min(0, min w), hi = max(0, max w);
 * s = fp16(fp32((hi - lo) / 15)); z = clamp(rint(-lo / s), 0, 15);
 * q = clamp(rint(w / s) + z, 0, 15); a group with s == 0 gets q = z = 0.
 * Writes codes [N][K], scale [N][K/G], zero [N][K/G].
 *
 * fmt == W4_NF4 ([NF4]): a = fp16(max |w|) per block of G; idx = the index i
 * minimizing |w - c_i * a| in fp64 over the 16 fp32 NormalFloat levels c_i
 * (lowest i on ties); a block with a == 0 gets idx = 7 (the zero level).
 * Writes codes [N][K] and the absmax into `scale`; `zero` must be NULL.
 *
 * rint is round-half-to-even.  Results are bit-exact functions of the input;
 * weights must be finite.  Codes are unpacked; see w4_pack.
 */
int w4_quantize(const float* wt, int K, int N, int G, int fmt,
                uint8_t* codes, uint16_t* scale, uint16_t* zero, void* stream);

/*
 * w4_pack -- pack codes [N][K] (values 0..15) into the tiled four-bit form
 * described under Layouts (N*K/2 bytes).  Four-bit storage is the 4x
 * reduction against fp16 noted on the [NF4] page.  Requires K % 128 == 0 and
 * N % 16 == 0.  Codes above 15 are masked to 4 bits.
 */
int w4_pack(const uint8_t* codes, int K, int N, uint8_t* packed, void* stream);

/*
 * w4_gemv -- decode-shaped product y[M][N] = x[M][K] . W', 1 <= M <= 32.
 *
 * Reads each packed weight once from HBM.  The group scale (and, for INT4, the
 * zero point) is applied to each group's partial sum after accumulation
 * ([MixPE]); NF4 levels come from a small on-chip table ([NF4]: codebook in
 * shared memory).  `ws`/`ws_bytes`: workspace of at least
 * w4_workspace_bytes(W4_OP_GEMV, M, K, N, G, fmt) bytes; when that is 0, ws may
 * be NULL.  Shapes whose activation slice does not fit on chip split K over
 * workgroups; the workspace then holds their fp32 partial sums
 * [S][M][N], which a second kernel on the same stream adds in slice order.
 * The workspace needs no initial contents (it is written before it is read).
 * Calls that overlap in time must not share a workspace.  Repeated calls give
 * bit-identical results.  Output y is fp16, rounded to nearest-even from fp32
 * accumulation.
 */
int w4_gemv(const uint16_t* x, int M, int K, int N,
            const uint8_t* packed, const uint16_t* scale, const uint16_t* zero,
            int G, int fmt, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/*
 * w4_gemv_noalloc -- w4_gemv for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels, plan and results (bit-identical to w4_gemv),
 * with no workspace argument.  Split-K partials go to a fixed 4 MiB device
 * array inside the library, one per device, held until the process ends; a
 * shape whose partials need more (w4_workspace_bytes(W4_OP_GEMV, ...) >
 * 4 MiB) returns W4_EWORKSPACE and enqueues nothing.  The array's address is
 * looked up on the first call on each device (no allocation).  Calls on one
 * device share that array: calls that overlap in time on one device (other
 * streams, other threads) race and must be ordered by the caller.  Arguments
 * and errors otherwise as for w4_gemv.
 */
int w4_gemv_noalloc(const uint16_t* x, int M, int K, int N,
                    const uint8_t* packed, const uint16_t* scale, const uint16_t* zero,
                    int G, int fmt, uint16_t* y, void* stream);

/*
 * w4_gemv_plan -- host-only introspection: the launch plan w4_gemv would use
 * for this shape and format on this thread right now (the W4_GEMV_*
 * environment overrides included).  Writes min(n_out, W4_GEMV_PLAN_FIELDS)
 * int64 values to out (host memory), in this order:
 *   0 kernel (0 = staged activations, 1 = direct operand loads),
 *   1 tile columns per wave, 2 token tiles of 16, 3 row waves,
 *   4 K waves, 5 K slices over workgroups, 6 staged units per thread,
 *   7 workgroups along N, 8 threads per workgroup, 9 dynamic LDS bytes,
 *   10 dynamic LDS budget, 11 static LDS bytes (for NF4 the level table:
 *      16 KB, or 64 KB where the plan runs one workgroup per CU and the
 *      LDS allows; W4_GEMV_LUT=16 keeps 16 KB), 12 workspace bytes,
 *   13 1 when the plan meets the kernels' bounds (threads <= 512, dynamic
 *      LDS within budget), else 0 -- w4_gemv refuses such a plan,
 *   14 weight tiles (staged kernel) or operand slots (direct kernel) each
 *      wave keeps in flight,
 *   15 1 when the direct kernel loads the activations whole rows at a time
 *      and reorders them through LDS, else 0.
 * Shape rules and errors as for w4_gemv; nothing touches a device.
 */
#define W4_GEMV_PLAN_FIELDS 16
int w4_gemv_plan(int M, int K, int N, int G, int fmt, int64_t* out, int n_out);

/*
 * w4_gemm -- prefill-shaped product y[M][N] = x[M][K] . W' for any M >= 1 on
 * fp16 matrix cores, in `mode` W4_DQ_F16 or W4_POSTSCALE (see w4_mode), for
 * either weight format.  Workspace is optional: when the output tiles alone
 * would not fill the GPU (e.g. M = 256, N = 8192), K is split over
 * workgroups if the caller passes at least
 * w4_workspace_bytes(W4_OP_GEMM, M, K, N, G, mode) bytes (16-byte aligned,
 * no initial contents needed: fp32 partials [S][M][N], added in slice order
 * by a second kernel on the same stream).  When the tiles fill the GPU but
 * leave a partial last round (tiles = q * CUs + r, 0 < r <= CUs / 2), the r
 * left-over tiles run as a second launch with K split over S workgroups each,
 * their fp32 partials [S][r][128][256] in the workspace, and a reduction
 * kernel writes their part of y.  With less workspace (or NULL) the product
 * runs as one launch.  Results do not depend on the split beyond fp32
 * rounding of the partial sums.
 */
int w4_gemm(const uint16_t* x, int M, int K, int N,
            const uint8_t* packed, const uint16_t* scale, const uint16_t* zero,
            int G, int fmt, int mode, uint16_t* y, void* ws, size_t ws_bytes,
            void* stream);

/*
 * w4_gemm_decomp -- Multi-Scale Dequant product ([MSD]): the fp16 activations
 * are split into `nslices` (1, 2 or 3) int8 slices with per-token fp32 scales,
 * and each slice is multiplied directly with the 4-bit integer weights on the
 * int8 matrix cores, with no conversion of the weights to a floating type.
 *
 * Decomposition, per token m, in fp64 with r = x: s_j = fp32(max|r| / 127);
 * A_j = clamp(rint(r / s_j), -127, 127); r -= s_j * A_j; a zero scale gives an
 * all-zero slice.  Products: D_j[m,g,n] = sum_{k in g} A_j[m,k] * (q[n,k] -
 * z[n,g]) exactly in int32; y[m,n] = sum_j s_j[m] * sum_g s[n,g] * D_j[m,g,n]
 * accumulated in fp32 and rounded to fp16.
 *
 * INT4 weights only: NF4 levels are not integers, so NF4 weights (zero ==
 * NULL) return W4_EUNSUPPORTED.  Also requires nslices * M * K < 4 GiB.
 * Optional outputs (NULL to skip): slices_out int8 [nslices][M][K] (row-major,
 * K contiguous); tok_scale_out fp32 [nslices][M]; acc_out int32
 * [nslices][M][K/G][N], the per-group integer accumulators (a debugging aid
 * for small shapes; it selects a slower kernel).
 * Workspace (required, 16-byte aligned, contents need not be initialised):
 * at least w4_workspace_bytes(W4_OP_GEMM_DECOMP, M, K, 0, G, nslices) bytes,
 * which hold the slices in the int8 matrix-core operand order and, when
 * tok_scale_out is NULL, the per-token scales.  w4_workspace_bytes with the
 * real N adds room for the fp32 partials of the tiles left over from the last
 * full round on the CUs, which then run with K split over workgroups (as in
 * w4_gemm; without that room they run unsplit).  Calls that overlap in time
 * must not share it.
 */
int w4_gemm_decomp(const uint16_t* x, int M, int K, int N,
                   const uint8_t* packed, const uint16_t* scale,
                   const uint16_t* zero, int G, int nslices, uint16_t* y,
                   int8_t* slices_out, float* tok_scale_out, int32_t* acc_out,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * w4_gemm_decomp_fixed -- two-slice Multi-Scale Dequant product ([MSD]) with
 * a fixed ratio between the slice scales, so that the two int8 products
 * combine exactly in integers before any conversion.
 *
 * The MSD abstract does not fix how the second scale is chosen; here it is
 * the first slice's step divided by 254.  Per token m, in fp64:
 * s_1 = fp32(max|x| / 127); A_1 = clamp(rint(x / s_1), -127, 127);
 * r_1 = x - s_1 A_1; A_2 = clamp(rint((254 r_1) / s_1), -127, 127).  Since
 * |r_1| <= s_1 / 2 the second slice never clamps in practice, and
 * |x - s_1 A_1 - (s_1 / 254) A_2| <= s_1 / 508.  Products: D_j as in
 * w4_gemm_decomp; E[m,g,n] = 254 D_1 + D_2 exactly in int32;
 * y[m,n] = (s_1[m] / 254) * sum_g s[n,g] * E[m,g,n], accumulated in fp32.
 *
 * Arguments, shapes, errors and workspace as for w4_gemm_decomp with
 * nslices = 2 (workspace: w4_workspace_bytes(W4_OP_GEMM_DECOMP, ..., 2));
 * tok_scale_out [2][M] receives s_1 and fp32(s_1 / 254); acc_out
 * [2][M][K/G][N] receives D_1 and D_2.
 */
int w4_gemm_decomp_fixed(const uint16_t* x, int M, int K, int N,
                         const uint8_t* packed, const uint16_t* scale,
                         const uint16_t* zero, int G, uint16_t* y,
                         int8_t* slices_out, float* tok_scale_out, int32_t* acc_out,
                         void* ws, size_t ws_bytes, void* stream);

/*
 * w4_gemm_decomp_fixed_fused -- the fixed-ratio Multi-Scale Dequant product
 * with the decomposition folded into the product's K loop ([MSD] Abstract:
 * the decomposition replaces the weight conversion on the product's critical
 * path).  A pre-pass over x computes only s_1 per token; each workgroup turns
 * every step's fp16 activation tile into the two int8 slices in LDS, so the
 * slices never reach HBM.  Codes, products and y are those of
 * w4_gemm_decomp_fixed, bit for bit (the slices are decided in fp32 by a
 * procedure proven to reproduce the fp64 decisions).
 *
 * Arguments, shapes and errors as for w4_gemm_decomp_fixed, without the
 * slices and integer-product outputs; requires M * K * 2 < 4 GiB.
 * tok_scale_out (optional, 16-byte aligned) fp32 [2][M] receives s_1 and
 * fp32(s_1 / 254).  Workspace (required, 16-byte aligned, contents need not
 * be initialised): at least w4_workspace_bytes(W4_OP_GEMM_DECOMP_FUSED, M, K,
 * 0, G, 0) bytes for the token scales; with the real N it adds room for the
 * fp32 partials of the left-over tiles, as for w4_gemm_decomp.  Calls that
 * overlap in time must not share it.
 */
int w4_gemm_decomp_fixed_fused(const uint16_t* x, int M, int K, int N,
                               const uint8_t* packed, const uint16_t* scale,
                               const uint16_t* zero, int G, uint16_t* y,
                               float* tok_scale_out, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * MXFP4 path ([MSD] Abstract: MXFP4 weights; the activations split into two
 * MXFP4 parts, each multiplied with the weights directly on the matrix cores).
 *
 * MXFP4 is the published OCP Microscaling element format E2M1 (sign, 2-bit
 * exponent with bias 1, 1-bit mantissa; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6;
 * codes 0..15 with bit 3 the sign) with one E8M0 scale byte s per 32
 * consecutive K positions (value 2^(s - 127)).  Scale rule (a reading: the
 * pages give none): the smallest e with max|v| <= 6 * 2^e over the block
 * (no element saturates), clamped to [-127, 127]; an all-zero block gets
 * e = -127.  Elements round to nearest, ties to the even mantissa; a zero
 * result has code 0.  All decisions are exact (fp64).
 */

/*
 * w4_quantize_mx -- W^T fp32 [N][K] (device, 4-byte aligned, K % 32 == 0) ->
 * codes u8 [N][K] (one E2M1 code per byte) and scales u8 [N][K/32] (E8M0).
 */
int w4_quantize_mx(const float* wt, int K, int N, uint8_t* codes, uint8_t* scale, void* stream);

/*
 * w4_pack_mx -- codes [N][K] -> packed [N*K/2] in 1 KB tiles of 16 rows x 128
 * K positions, tile (nb, kb) at byte (nb*K/128 + kb)*1024; in a tile, the 16
 * bytes at 16*(16j + r) hold row r's positions 128kb + 32j .. + 31, two per
 * byte, low nibble first (the operand order of the block-scaled fp4 product).
 * Requires K % 128 == 0, N % 16 == 0; packed 16-byte aligned.
 */
int w4_pack_mx(const uint8_t* codes, int K, int N, uint8_t* packed, void* stream);

/*
 * w4_gemm_mx -- y[M][N] fp16 = x . W' with MXFP4 weights (packed by
 * w4_pack_mx, scales [N][K/32]) and the activations split into `nslices`
 * (1 or 2) MXFP4 slices: slice 1 = MXFP4(x), slice 2 = MXFP4(x - slice 1),
 * per token and block of 32, in fp64.  Each slice meets the weights on the
 * block-scaled fp4 matrix cores, which apply both E8M0 scales; the products
 * accumulate in fp32.  Two slices: at most 2^(e1 - 3) error per element of a
 * block, which is 1/64 of 2^(e1 + 3), the power of two above the first
 * slice's largest value 6 * 2^e1 ([MSD]'s 1/64 per block), and below
 * amax/24 (e1 the first slice's exponent, amax the block's max).
 *
 * Requires K % 128 == 0, N % 16 == 0, x and y 16-byte aligned, operands below
 * 4 GiB.  Optional outputs (NULL to skip): slices_out u8 [nslices][M][K/2]
 * (packed, low nibble first), scales_out u8 [nslices][M][K/32].  Workspace
 * (required, 16-byte aligned, no initial contents): at least
 * w4_workspace_bytes(W4_OP_GEMM_MX, M, K, 0, 32, nslices) bytes for the
 * slices and their scales; w4_workspace_bytes with the real N adds room for
 * the split-K partials of the left-over tiles, as for w4_gemm_decomp.
 */
int w4_gemm_mx(const uint16_t* x, int M, int K, int N, const uint8_t* packed,
               const uint8_t* scale, int nslices, uint16_t* y, uint8_t* slices_out,
               uint8_t* scales_out, void* ws, size_t ws_bytes, void* stream);

/*
 * w4_attn_decode_msd -- decode attention (one query token per head) over an
 * INT4 KV cache with Multi-Scale Dequant on both products ([MSD] Abstract:
 * the cache stays quantized and the other operand of each product is
 * decomposed, which cuts the cache's HBM traffic).
 *
 * q: fp16 [B][Hq][d] device, d = 128.  Query head g of a batch row uses
 *   key/value head g / (Hq/Hkv) (grouped-query attention, Hq/Hkv <= 16).
 * K cache, per (b, h): the [L][d] matrix quantized per token (w4_quantize
 *   with G = 128 on it as W^T [N=L][K=d]) and packed by w4_pack;
 *   k_packed [B][Hkv][L*d/2], k_scale and k_zero fp16 [B][Hkv][L].
 * V cache, per (b, h): quantized per token the same way, its codes
 *   transposed to [d][L] and packed by w4_pack (as W^T [N=d][K=L]);
 *   vt_packed [B][Hkv][d*L/2], v_scale and v_zero fp16 [B][Hkv][L].
 * out: fp16 [B][Hq][d].  L must be a multiple of 256.
 *
 * Computation: the queries are split into two int8 slices per head
 * (w4_gemm_decomp's decomposition); scores = sK[t] sum_j s_j (A_j . (qK[t] -
 * zK[t])) / sqrt(d) with exact int32 products; softmax per block of 256
 * positions (max m_c, sum l_c of exp(score - m_c)); w = exp(score - m_c) *
 * sV[t] is split per head and block into two int8 slices (B_j, r_j, same
 * rule), o_c = sum_j r_j sum_t B_j (qV[t] - zV[t]) exactly in int32; the
 * blocks are combined as sum_c e^(m_c - m) o_c / sum_c e^(m_c - m) l_c.
 * Workspace (required, 16-byte aligned, no initial contents):
 * w4_workspace_bytes(W4_OP_ATTN_MSD, B, Hq, L, 0, 0) bytes.
 */
int w4_attn_decode_msd(const uint16_t* q, int B, int Hq, int Hkv, int L, int d,
                       const uint8_t* k_packed, const uint16_t* k_scale, const uint16_t* k_zero,
                       const uint8_t* vt_packed, const uint16_t* v_scale, const uint16_t* v_zero,
                       uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * w4_salient_select -- the k salient input channels of a decode step, for
 * residual compensation ([DecDEC] Abstract: salient channels are those where
 * the current activations have outliers, chosen anew at every step).
 *
 * x: fp16 [M][K] device, 2-byte aligned.  Channel c scores max_m |x[m,c]|
 * (NaN inputs give an unspecified choice).  idx: int32 [k] device, receives
 * the k highest-scoring channels ordered by score (descending) and, among
 * equal scores, by channel (ascending) -- a unique order.  Requires
 * 1 <= K <= 32768 and 0 <= k <= min(K, 1024); k = 0 enqueues nothing.
 */
int w4_salient_select(const uint16_t* x, int M, int K, int k, int32_t* idx, void* stream);

/*
 * w4_residual_correct -- adds the residual of the picked channels to a
 * quantized product ([DecDEC] Abstract: the residual matrix, full-precision
 * minus quantized weights, is kept in host memory and fetched only for the
 * salient channels):  y[m,n] = fp16(y[m,n] + sum_j x[m,idx[j]] * R[idx[j],n]),
 * the sum in fp32.
 *
 * x: fp16 [M][K] device (the step's activations), 1 <= M <= 32.
 * resid: fp16 [K][N] (row c = channel c's residuals for every output),
 *   16-byte aligned, in pinned host memory (hipHostMalloc; read by the device
 *   over the host link, nothing is copied ahead) or in device memory;
 *   pageable host memory returns W4_EINVAL.  Caller-owned.
 * idx: int32 [k] device (e.g. from w4_salient_select); entries outside
 *   [0, K) are skipped.  y: fp16 [M][N] device, updated in place, 16-byte
 *   aligned.  Requires N % 8 == 0.  k = 0 enqueues nothing.
 */
int w4_residual_correct(const uint16_t* x, int M, int K, int N, const uint16_t* resid,
                        const int32_t* idx, int k, uint16_t* y, void* stream);

/*
 * w4_residual_correct_f32 -- the correction of w4_residual_correct, stored
 * instead of added: c[m,n] = sum_j x[m,idx[j]] * R[idx[j],n] in fp32 (every
 * element of c is written; k = 0 writes zeros).  It does not read the
 * product, so it can run on a second stream beside the GEMV that writes y
 * ([DecDEC] Abstract: the residual fetch is meant to add little to the
 * step's time); w4_residual_apply then adds c to y.  The two calls leave y
 * bit-identical to w4_residual_correct on the same y.
 *
 * x, resid, idx, M, K, N, k: as for w4_residual_correct (k = 0 still
 * launches).  c: fp32 [M][N] device, 16-byte aligned, written.
 */
int w4_residual_correct_f32(const uint16_t* x, int M, int K, int N, const uint16_t* resid,
                            const int32_t* idx, int k, float* c, void* stream);

/*
 * w4_residual_apply -- y[m,n] = fp16(y[m,n] + c[m,n]) for a correction from
 * w4_residual_correct_f32.  c: fp32 [M][N], y: fp16 [M][N], both device and
 * 16-byte aligned; N % 8 == 0.
 */
int w4_residual_apply(const float* c, int M, int N, uint16_t* y, void* stream);

/*
 * w4_salient_correct -- w4_salient_select followed by w4_residual_correct in
 * one launch ([DecDEC] Abstract: salient channels chosen anew at every step,
 * their residual rows fetched from host memory).  The picks and y are
 * exactly those of the two calls; idx receives the picks as
 * w4_salient_select writes them.
 *
 * x: fp16 [M][K] device, 1 <= M <= 32, 1 <= K <= 32768.  resid, y: as for
 * w4_residual_correct (N % 8 == 0).  idx: int32 [k] device, written.
 * Requires 0 <= k <= min(K, 1024); k = 0 enqueues nothing.  Every workgroup
 * of the launch makes the (deterministic) selection itself, so the call
 * needs no workspace.
 */
int w4_salient_correct(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k,
                       int32_t* idx, uint16_t* y, void* stream);

/*
 * w4_salient_correct_f32 -- w4_salient_select followed by
 * w4_residual_correct_f32 in one launch: the picks go to idx and the
 * correction is stored to c (fp32 [M][N], every element written; k = 0
 * writes zeros and still launches), for w4_residual_apply.  Arguments and
 * limits as for w4_salient_correct, with c (device, 16-byte aligned) in place
 * of y.
 */
int w4_salient_correct_f32(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k,
                           int32_t* idx, float* c, void* stream);

/*
 * w4_workspace_bytes -- bytes of workspace an entry point needs for the given
 * shape.  `fmt_or_mode`: the w4_fmt for W4_OP_GEMV, the w4_mode for
 * W4_OP_GEMM, nslices for W4_OP_GEMM_DECOMP and W4_OP_GEMM_MX.  Host-only;
 * returns 0 for ops that need none and (size_t)-1 for an invalid op.  The
 * split-K room of the matrix-core products depends on the current device's
 * CU count (none when no device is visible); N < 16 gives the minimum for
 * W4_OP_GEMM_DECOMP and W4_OP_GEMM_MX.
 */
size_t w4_workspace_bytes(int op, int M, int K, int N, int G, int fmt_or_mode);

/*
 * w4_stream_read -- a plain read of a device buffer, the measured HBM read
 * ceiling the weight-streaming kernels are compared with (not part of the
 * method).  Every 16-byte piece of buf is loaded once with a non-temporal
 * load, as the GEMV loads its weight tiles, and every 32-bit word is XORed
 * into one of the eight device words xor_acc[0], xor_acc[64], ...,
 * xor_acc[448] (spread so that the folds do not serialize on one address;
 * zero them first: their XOR is then the buffer's XOR).  buf 16-byte aligned
 * device memory, bytes a multiple of 16 (0: nothing happens); xor_acc 4-byte
 * aligned device memory of at least W4_STREAM_READ_ACC_WORDS words.  Errors:
 * W4_EINVAL for a null or misaligned pointer or a byte count that is not a
 * multiple of 16.
 */
#define W4_STREAM_READ_ACC_WORDS 449
int w4_stream_read(const void* buf, size_t bytes, uint32_t* xor_acc, void* stream);

/*
 * w4_mfma_rate -- the matrix-core issue rate, the measured ceiling the
 * prefill products are compared with beside the nominal dense peak (not part
 * of the method).  Launches `workgroups` workgroups of 512 threads (8 waves,
 * two per SIMD, as the prefill products run); every wave issues iters x 8
 * independent 16 x 16 products -- kind 0: v_mfma_f32_16x16x32_f16 (16384
 * flops each), kind 1: v_mfma_i32_16x16x64_i8 (32768 ops each) -- and, with
 * each product, `valu` independent fp32 FMAs (0, 1, 2, 3, 4, 6 or 8).  No
 * memory traffic besides the results: sink (device, workgroups x 512 floats)
 * receives a per-thread sum of the accumulators, and ticks (device, 2 words
 * per wave, or null) receives each wave's elapsed shader-clock ticks
 * (s_memtime) and 100 MHz real-time ticks (s_memrealtime) around its loop,
 * whose ratio is the clock the part ran at.  96 KB of LDS are reserved per
 * workgroup (and not used), so one workgroup runs per CU.  Errors: W4_EINVAL for another
 * kind or valu, workgroups or iters below 1, a null sink, or a misaligned
 * pointer.
 */
int w4_mfma_rate(int kind, int valu, int workgroups, int iters, float* sink, unsigned long long* ticks,
                 void* stream);

/* Host-only: copies the library's 16 fp32 NF4 levels into out16 (host). */
int w4_nf4_levels(float* out16);

/* Host-only: static text for a w4_status value. */
const char* w4_status_str(int status);

/* Host-only: message of the last failed call on this thread ("" if none). */
const char* w4_last_error(void);

/* Host-only: library version string. */
const char* w4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W4_H_ */

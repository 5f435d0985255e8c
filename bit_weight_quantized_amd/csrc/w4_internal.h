// Internal declarations shared by the library's translation units (not part
// of the public ABI; see include/w4.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4 {

// Records `msg` as this thread's last error and returns `status`.
int fail(int status, const char* fmt, ...);

// Clears this thread's last error (every entry point starts with it).
void clear_error();

// Argument checks shared by the entry points: each returns W4_OK or a
// negative w4_status with the error text recorded.
bool aligned16(const void* p);
int check_matmul_shape(const char* fn, int M, int K, int N, int G);
int check_weights(const char* fn, const uint8_t* packed, const uint16_t* scale, const uint16_t* zero, int fmt);
int check_io(const char* fn, const void* x, const void* y);
// w4_gemv's rules: the above plus 1 <= M <= 32.
int check_gemv_args(const char* fn, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                    const uint16_t* scale, const uint16_t* zero, int G, int fmt, const uint16_t* y);

// Maps the last HIP launch error to W4_EHIP (recording its text) or W4_OK.
int check_launch(const char* what);

// Allows kernel `fn` up to `bytes` of dynamic LDS on the current device (once
// per kernel and device); W4_OK, or W4_EHIP with the error text recorded.
int allow_dynamic_lds(const void* fn, int bytes, const char* what);

// ---- launchers (host side); arguments are validated by the caller ----
int launch_quantize_int4(const float* wt, int K, int N, int G, uint8_t* codes,
                         uint16_t* scale, uint16_t* zero, hipStream_t s);
int launch_quantize_nf4(const float* wt, int K, int N, int G, uint8_t* codes,
                        uint16_t* absmax, hipStream_t s);
int launch_pack(const uint8_t* codes, int K, int N, uint8_t* packed, hipStream_t s);

// Launch shape of the GEMV: token tiles (mt), row waves and K waves per
// workgroup (nwr, nwk), K slices over workgroups (s), staged activation units
// per thread (xu), grid rows, the LDS row pitch of each wave's scale block,
// the bytes of staged activations, dynamic LDS and workspace bytes (fp32
// split-K partials).
// kind 1 is the direct variant: cols tile columns per wave, no staging.
// ring: weight tiles (staged) or operand slots (direct) in flight per wave.
// vs: the staged kernel fetches its workgroup's scale block with 16-byte loads.
struct GemvPlan {
  int kind, cols, mt, nwr, nwk, s, xu, row_blocks, sc_pitch, x_bytes, ring, vs, xl, xl_off;
  int lut;  // NF4 table copies in LDS (16 or 64)
  size_t lds_bytes, ws_bytes;
};
GemvPlan plan_gemv(int M, int K, int N, int G, int fmt);
// Bounds every GEMV plan must meet: at most 512 threads per workgroup (the
// kernels' launch bound) and dynamic LDS within gemv_lds_budget (the static
// LDS, gemv_static_lds, comes on top).  check_gemv_plan returns 0 or a
// negative w4_status with the error text recorded.
size_t gemv_lds_budget(int fmt);
size_t gemv_static_lds(int fmt);
// the same for a given plan (its NF4 table size)
size_t gemv_plan_lds_budget(const GemvPlan& c, int fmt);
size_t gemv_plan_static_lds(const GemvPlan& c, int fmt);
int gemv_plan_threads(const GemvPlan& c);
int check_gemv_plan(const GemvPlan& c, int fmt);
int launch_gemv(const GemvPlan& plan, const uint16_t* x, int M, int K, int N,
                const uint8_t* packed, const uint16_t* scale, const uint16_t* zero,
                int G, int fmt, uint16_t* y, void* ws, hipStream_t s);

// Row blocks per group in the matrix-core kernels' tile order (see tile_of;
// W4_GEMM_GM overrides the default for sweeps).
int gemm_group_rows();

// Matrix-core GEMMs run one workgroup per CU.  With tiles = q C + r (C CUs,
// 0 < r <= C / 2), the q C tiles run as one launch and the r left over as a
// second launch with each tile's K steps split over S workgroups: fp32
// partials [S][r][bm][bn] (`bytes`), then tail_reduce writes those tiles of
// y.  S = 1: no tail launch.  W4_GEMM_TAIL=0 turns it off.
struct TailPlan {
  long main;  // tiles of the first launch (places [0, main) of the walk)
  int r, S;
  size_t bytes;
};
int device_cus();  // compute units of the current device, 0 when unknown
TailPlan plan_tail(long tiles, int KT, int bm, int bn);
int launch_tail_reduce(const float* tpart, const TailPlan& tp, int bm, int bn, int tiles_m, int tiles_n, int gm,
                       int M, int N, uint16_t* y, hipStream_t s);

// fp16 GEMM: K slices over workgroups (1 when the grid already fills the
// chip) and the fp32 partial workspace that takes ([S][M][N] when S > 1,
// else the tail's partials).
int gemm_split(int M, int K, int N);
size_t gemm_workspace_bytes(int M, int K, int N);
// Launches the fp16 GEMM; with ws_bytes < gemm_workspace_bytes it runs unsplit
// (and without a tail launch).
int launch_gemm(const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                const uint16_t* scale, const uint16_t* zero, int G, int fmt,
                int mode, uint16_t* y, void* ws, size_t ws_bytes, hipStream_t s);
// y[i] = fp16(sum over k < S of partial[k * MN + i]) in slice order.
int launch_reduce_partials(const float* partial, int S, long MN, uint16_t* y, hipStream_t s);

// Workspace of the decomposed product: int8 slices [nslices][M][K] in the
// matrix-core operand layout (256-byte aligned), then fp32 token scales
// [nslices][M].
size_t decomp_workspace_bytes(int M, int K, int G, int nslices);
// Optional room for the tail's partials after that (the product runs without
// a tail launch when the workspace does not hold it).
size_t decomp_tail_bytes(int M, int K, int N, int G, int nslices);
// Decomposition: operand-layout slices, plus the plain layout when
// slices_out is non-null.  nslices 1..3 with adaptive scales, or (fixed) two
// slices with s_2 = s_1 / 254.
int launch_decompose(const uint16_t* x, int M, int K, int nslices, bool fixed, int8_t* slices_op,
                     int8_t* slices_out, float* tok_scale, hipStream_t s);
int launch_gemm_decomp(const uint16_t* x, int M, int K, int N,
                       const uint8_t* packed, const uint16_t* scale,
                       const uint16_t* zero, int G, int nslices, bool fixed, uint16_t* y,
                       int8_t* slices_op, int8_t* slices_out, float* tok_scale,
                       int32_t* acc_out, float* tpart, size_t tpart_bytes, hipStream_t s);
// Fixed-ratio product with the decomposition inside the product's K loop:
// fp32 token scales [2][M] (s_1, s_1 / 254) from a row-absmax pre-pass, then
// one product launch (plus the tail, as for launch_gemm_decomp; its partials
// need decomp_tail_bytes(M, K, N, G, 2)).
size_t decomp_fused_workspace_bytes(int M);
int launch_gemm_decomp_fused(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                             const uint16_t* zero, int G, uint16_t* y, float* tok_scale, float* tpart,
                             size_t tpart_bytes, hipStream_t s);

// Residual compensation: the k salient channels of x (k <= kSelMaxTop,
// K <= kSelMaxK), and y += x[:, idx] . R[idx, :] with R fp16 [K][N] in memory
// the device can read (M <= 32).
constexpr int kSelMaxK = 32768;
constexpr int kSelMaxTop = 1024;
int launch_salient_select(const uint16_t* x, int M, int K, int k, int32_t* idx, hipStream_t s);
int launch_residual_correct(const uint16_t* x, int M, int K, int N, const uint16_t* resid, const int32_t* idx,
                            int k, uint16_t* y, hipStream_t s);
int launch_residual_correct_f32(const uint16_t* x, int M, int K, int N, const uint16_t* resid, const int32_t* idx,
                                int k, float* c, hipStream_t s);
int launch_residual_apply(const float* c, int M, int N, uint16_t* y, hipStream_t s);
int launch_salient_correct_f32(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k, int32_t* idx,
                               float* c, hipStream_t s);
int launch_salient_correct(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k, int32_t* idx,
                           uint16_t* y, hipStream_t s);

// MXFP4 weights (codes one per byte, E8M0 scales [N][K/32]), their packing
// into 1 KB tiles, and the MXFP4 product with the activations split into
// nslices (1 or 2) MXFP4 slices; workspace: slices [ns][M][K/2], then scales
// [ns][M][K/32], each 256-byte aligned.
int launch_quantize_mx(const float* wt, int K, int N, uint8_t* codes, uint8_t* scale, hipStream_t s);
int launch_pack_mx(const uint8_t* codes, int K, int N, uint8_t* packed, hipStream_t s);
size_t mx_workspace_bytes(int M, int K, int nslices);
size_t mx_tail_bytes(int M, int K, int N, int nslices);  // optional, after the above
int launch_gemm_mx(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint8_t* wscale, int nslices,
                   uint16_t* y, uint8_t* slices_out, uint8_t* scales_out, void* ws, size_t ws_bytes, hipStream_t s);

// Decode attention over an INT4 KV cache with MSD on both products (head
// dimension 128, L % 256 == 0, Hq / Hkv <= 16); workspace: query slices and
// scales, then per-chunk partial outputs and (max, sum).
size_t attn_workspace_bytes(int B, int Hq, int L);
int launch_attn_msd(const uint16_t* q, int B, int Hq, int Hkv, int L, const uint8_t* kp, const uint16_t* ks,
                    const uint16_t* kz, const uint8_t* vtp, const uint16_t* vs, const uint16_t* vz, uint16_t* out,
                    void* ws, hipStream_t s);

// The 16 NF4 levels as fp32 bit patterns (host copy).
extern const uint32_t kNf4LevelBits[16];

// Plain read of bytes / 16 16-byte pieces, XOR-folded into *acc.
int launch_stream_read(const void* buf, size_t bytes, uint32_t* acc, hipStream_t s);

// Independent matrix-core products (kind 0 fp16, 1 int8) with valu fp32 FMAs
// each, iters rounds of 8 per wave, 512 threads per workgroup.
int launch_mfma_rate(int kind, int valu, int workgroups, int iters, float* sink, unsigned long long* ticks,
                     hipStream_t s);

}  // namespace w4

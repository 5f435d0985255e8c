// Host side of the C ABI declared in include/w4.h: argument validation,
// status codes, the thread-local error text and dispatch to the launchers.
#include "../../include/w4.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <set>
#include <tuple>

#include "w4_internal.h"

#include <cstdlib>

namespace w4 {

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

void clear_error() { g_last_error[0] = '\0'; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_group(int G) { return G == 64 || G == 128; }

// Shape rules shared by the matmul entry points.
int check_matmul_shape(const char* fn, int M, int K, int N, int G) {
  if (M < 1) return fail(W4_EINVAL, "%s: M must be >= 1 (got %d)", fn, M);
  if (K < 1 || N < 1) return fail(W4_EINVAL, "%s: K and N must be >= 1 (got K=%d N=%d)", fn, K, N);
  if (!valid_group(G)) return fail(W4_EINVAL, "%s: G must be 64 or 128 (got %d)", fn, G);
  if (K % G != 0) return fail(W4_EINVAL, "%s: K=%d is not a multiple of G=%d", fn, K, G);
  if (K % 128 != 0) return fail(W4_EINVAL, "%s: K=%d is not a multiple of 128 (the weight tile)", fn, K);
  if (N % 16 != 0) return fail(W4_EINVAL, "%s: N=%d is not a multiple of 16", fn, N);
  if ((uint64_t)(N + 16) * (uint64_t)(K / 2) >= (1ull << 32))
    return fail(W4_EINVAL, "%s: packed weights of %d x %d exceed the 4 GiB addressable per matrix", fn, N, K);
  return W4_OK;
}

int check_weights(const char* fn, const uint8_t* packed, const uint16_t* scale,
                  const uint16_t* zero, int fmt) {
  if (fmt != W4_INT4_ASYM && fmt != W4_NF4) return fail(W4_EINVAL, "%s: unknown fmt %d", fn, fmt);
  if (!packed || !scale) return fail(W4_EINVAL, "%s: packed and scale must be non-null", fn);
  if (fmt == W4_INT4_ASYM && !zero) return fail(W4_EINVAL, "%s: INT4 weights need a zero-point array", fn);
  if (fmt == W4_NF4 && zero) return fail(W4_EINVAL, "%s: NF4 weights take zero == NULL", fn);
  if (!aligned16(packed) || !aligned16(scale) || (zero && !aligned16(zero)))
    return fail(W4_EINVAL, "%s: weight pointers must be 16-byte aligned", fn);
  return W4_OK;
}

int check_io(const char* fn, const void* x, const void* y) {
  if (!x || !y) return fail(W4_EINVAL, "%s: x and y must be non-null", fn);
  if (!aligned16(x) || !aligned16(y)) return fail(W4_EINVAL, "%s: x and y must be 16-byte aligned", fn);
  return W4_OK;
}

int check_gemv_args(const char* fn, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                    const uint16_t* scale, const uint16_t* zero, int G, int fmt, const uint16_t* y) {
  int st;
  if ((st = check_matmul_shape(fn, M, K, N, G)) != W4_OK) return st;
  if (M > 32) return fail(W4_EINVAL, "%s: M must be <= 32 (got %d); use w4_gemm", fn, M);
  if ((st = check_weights(fn, packed, scale, zero, fmt)) != W4_OK) return st;
  return check_io(fn, x, y);
}

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(W4_EHIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return W4_OK;
}

int allow_dynamic_lds(const void* fn, int bytes, const char* what) {
  static std::mutex mu;
  static std::set<std::tuple<const void*, int, int>> done;  // (kernel, device, bytes)
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(W4_EHIP, "%s: hipGetDevice: %s", what, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({fn, dev, bytes})) return W4_OK;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return fail(W4_EHIP, "%s: cannot reserve %d bytes of LDS: %s", what, bytes, hipGetErrorString(e));
  done.insert({fn, dev, bytes});
  return W4_OK;
}

int gemm_group_rows() {
  static const int gm = [] {
    const char* e = std::getenv("W4_GEMM_GM");
    const int v = e && *e ? std::atoi(e) : 4;
    return v >= 1 && v <= 64 ? v : 4;
  }();
  return gm;
}

const uint32_t kNf4LevelBits[16] = {
    0xbf800000u, 0xbf3239b1u, 0xbf066b2eu, 0xbeca329eu, 0xbe91a24bu, 0xbe3d353du,
    0xbdba7869u, 0x00000000u, 0x3da2fb01u, 0x3e24cadfu, 0x3e7c04dau, 0x3ead0336u,
    0x3ee1a4b5u, 0x3f1007a9u, 0x3f3913b0u, 0x3f800000u};

namespace {

int gemm_decomp_checked(const char* fn, const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                        const uint16_t* scale, const uint16_t* zero, int G, int nslices, bool fixed, uint16_t* y,
                        int8_t* slices_out, float* tok_scale_out, int32_t* acc_out, void* ws, size_t ws_bytes,
                        void* stream) {
  g_last_error[0] = '\0';
  int st;
  if ((st = check_matmul_shape(fn, M, K, N, G)) != W4_OK) return st;
  if (nslices < 1 || nslices > 3) return fail(W4_EINVAL, "%s: nslices must be 1, 2 or 3 (got %d)", fn, nslices);
  if (packed && scale && !zero)
    return fail(W4_EUNSUPPORTED, "%s: needs INT4 weights (zero != NULL); NF4 levels are not integers", fn);
  if ((st = check_weights(fn, packed, scale, zero, W4_INT4_ASYM)) != W4_OK) return st;
  if ((st = check_io(fn, x, y)) != W4_OK) return st;
  if ((slices_out && !aligned16(slices_out)) || (tok_scale_out && !aligned16(tok_scale_out)) ||
      (acc_out && !aligned16(acc_out)))
    return fail(W4_EINVAL, "%s: optional outputs must be 16-byte aligned", fn);
  const size_t need = decomp_workspace_bytes(M, K, G, nslices);
  if (!ws || ws_bytes < need)
    return fail(W4_EWORKSPACE, "%s: workspace of %zu bytes required (got %zu)", fn, need, ws_bytes);
  if (!aligned16(ws)) return fail(W4_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  char* base = static_cast<char*>(ws);
  const size_t slice_bytes = ((size_t)nslices * M * K + 255) / 256 * 256;
  int8_t* sl_op = reinterpret_cast<int8_t*>(base);
  float* ts = tok_scale_out ? tok_scale_out : reinterpret_cast<float*>(base + slice_bytes);
  // the tail's partials, when the workspace holds them after the slices and scales
  float* tpart = ws_bytes > need ? reinterpret_cast<float*>(base + need) : nullptr;
  return launch_gemm_decomp(x, M, K, N, packed, scale, zero, G, nslices, fixed, y, sl_op, slices_out, ts, acc_out,
                            tpart, ws_bytes - need, (hipStream_t)stream);
}

}  // namespace

}  // namespace w4

using namespace w4;

extern "C" {

int w4_quantize(const float* wt, int K, int N, int G, int fmt, uint8_t* codes,
                uint16_t* scale, uint16_t* zero, void* stream) {
  g_last_error[0] = '\0';
  if (K < 1 || N < 1) return fail(W4_EINVAL, "w4_quantize: K and N must be >= 1 (got K=%d N=%d)", K, N);
  if (!valid_group(G)) return fail(W4_EINVAL, "w4_quantize: G must be 64 or 128 (got %d)", G);
  if (K % G != 0) return fail(W4_EINVAL, "w4_quantize: K=%d is not a multiple of G=%d", K, G);
  if (!wt || !codes || !scale) return fail(W4_EINVAL, "w4_quantize: wt, codes and scale must be non-null");
  if (fmt == W4_INT4_ASYM) {
    if (!zero) return fail(W4_EINVAL, "w4_quantize: INT4 needs a zero-point array");
    return launch_quantize_int4(wt, K, N, G, codes, scale, zero, (hipStream_t)stream);
  }
  if (fmt == W4_NF4) {
    if (zero) return fail(W4_EINVAL, "w4_quantize: NF4 takes zero == NULL");
    return launch_quantize_nf4(wt, K, N, G, codes, scale, (hipStream_t)stream);
  }
  return fail(W4_EINVAL, "w4_quantize: unknown fmt %d", fmt);
}

int w4_pack(const uint8_t* codes, int K, int N, uint8_t* packed, void* stream) {
  g_last_error[0] = '\0';
  if (K < 1 || N < 1) return fail(W4_EINVAL, "w4_pack: K and N must be >= 1 (got K=%d N=%d)", K, N);
  if (K % 128 != 0) return fail(W4_EINVAL, "w4_pack: K=%d is not a multiple of 128 (the weight tile)", K);
  if (N % 16 != 0) return fail(W4_EINVAL, "w4_pack: N=%d is not a multiple of 16 (the weight tile)", N);
  if (!codes || !packed) return fail(W4_EINVAL, "w4_pack: codes and packed must be non-null");
  if (!aligned16(codes) || !aligned16(packed)) return fail(W4_EINVAL, "w4_pack: pointers must be 16-byte aligned");
  return launch_pack(codes, K, N, packed, (hipStream_t)stream);
}

int w4_gemv(const uint16_t* x, int M, int K, int N, const uint8_t* packed,
            const uint16_t* scale, const uint16_t* zero, int G, int fmt, uint16_t* y,
            void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  int st;
  if ((st = check_gemv_args("w4_gemv", x, M, K, N, packed, scale, zero, G, fmt, y)) != W4_OK) return st;
  const GemvPlan plan = plan_gemv(M, K, N, G, fmt);
  if (plan.ws_bytes > 0) {
    if (!ws || ws_bytes < plan.ws_bytes)
      return fail(W4_EWORKSPACE, "w4_gemv: workspace of %zu bytes required (got %zu)", plan.ws_bytes, ws_bytes);
    if (!aligned16(ws)) return fail(W4_EINVAL, "w4_gemv: workspace must be 16-byte aligned");
  }
  return launch_gemv(plan, x, M, K, N, packed, scale, zero, G, fmt, y, ws, (hipStream_t)stream);
}

int w4_gemv_plan(int M, int K, int N, int G, int fmt, int64_t* out, int n_out) {
  g_last_error[0] = '\0';
  int st;
  if ((st = check_matmul_shape("w4_gemv_plan", M, K, N, G)) != W4_OK) return st;
  if (M > 32) return fail(W4_EINVAL, "w4_gemv_plan: M must be <= 32 (got %d)", M);
  if (fmt != W4_INT4_ASYM && fmt != W4_NF4) return fail(W4_EINVAL, "w4_gemv_plan: unknown fmt %d", fmt);
  if (!out || n_out < 0) return fail(W4_EINVAL, "w4_gemv_plan: out must be non-null");
  const GemvPlan c = plan_gemv(M, K, N, G, fmt);
  const int64_t v[W4_GEMV_PLAN_FIELDS] = {c.kind,
                                          c.cols,
                                          c.mt,
                                          c.kind == 1 ? 1 : c.nwr,
                                          c.nwk,
                                          c.s,
                                          c.xu,
                                          c.row_blocks,
                                          gemv_plan_threads(c),
                                          (int64_t)c.lds_bytes,
                                          (int64_t)gemv_plan_lds_budget(c, fmt),
                                          (int64_t)gemv_plan_static_lds(c, fmt),
                                          (int64_t)c.ws_bytes,
                                          check_gemv_plan(c, fmt) == 0 ? 1 : 0,
                                          c.ring,
                                          c.kind == 1 ? c.xl : 0};
  for (int i = 0; i < n_out && i < W4_GEMV_PLAN_FIELDS; ++i) out[i] = v[i];
  g_last_error[0] = '\0';
  return W4_OK;
}

int w4_gemm(const uint16_t* x, int M, int K, int N, const uint8_t* packed,
            const uint16_t* scale, const uint16_t* zero, int G, int fmt, int mode,
            uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  int st;
  if ((st = check_matmul_shape("w4_gemm", M, K, N, G)) != W4_OK) return st;
  if (mode != W4_DQ_F16 && mode != W4_POSTSCALE) return fail(W4_EINVAL, "w4_gemm: unknown mode %d", mode);
  if ((st = check_weights("w4_gemm", packed, scale, zero, fmt)) != W4_OK) return st;
  if ((st = check_io("w4_gemm", x, y)) != W4_OK) return st;
  if (ws && ws_bytes >= gemm_workspace_bytes(M, K, N) && !aligned16(ws))
    return fail(W4_EINVAL, "w4_gemm: workspace must be 16-byte aligned");
  return launch_gemm(x, M, K, N, packed, scale, zero, G, fmt, mode, y, ws, ws_bytes, (hipStream_t)stream);
}

int w4_gemm_decomp(const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                   const uint16_t* scale, const uint16_t* zero, int G, int nslices,
                   uint16_t* y, int8_t* slices_out, float* tok_scale_out, int32_t* acc_out,
                   void* ws, size_t ws_bytes, void* stream) {
  return gemm_decomp_checked("w4_gemm_decomp", x, M, K, N, packed, scale, zero, G, nslices, false, y, slices_out,
                             tok_scale_out, acc_out, ws, ws_bytes, stream);
}

int w4_gemm_decomp_fixed(const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                         const uint16_t* scale, const uint16_t* zero, int G, uint16_t* y,
                         int8_t* slices_out, float* tok_scale_out, int32_t* acc_out,
                         void* ws, size_t ws_bytes, void* stream) {
  return gemm_decomp_checked("w4_gemm_decomp_fixed", x, M, K, N, packed, scale, zero, G, 2, true, y, slices_out,
                             tok_scale_out, acc_out, ws, ws_bytes, stream);
}

int w4_gemm_decomp_fixed_fused(const uint16_t* x, int M, int K, int N, const uint8_t* packed,
                               const uint16_t* scale, const uint16_t* zero, int G, uint16_t* y,
                               float* tok_scale_out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "w4_gemm_decomp_fixed_fused";
  g_last_error[0] = '\0';
  int st;
  if ((st = check_matmul_shape(fn, M, K, N, G)) != W4_OK) return st;
  if (packed && scale && !zero)
    return fail(W4_EUNSUPPORTED, "%s: needs INT4 weights (zero != NULL); NF4 levels are not integers", fn);
  if ((st = check_weights(fn, packed, scale, zero, W4_INT4_ASYM)) != W4_OK) return st;
  if ((st = check_io(fn, x, y)) != W4_OK) return st;
  if (tok_scale_out && !aligned16(tok_scale_out))
    return fail(W4_EINVAL, "%s: tok_scale_out must be 16-byte aligned", fn);
  const size_t need = decomp_fused_workspace_bytes(M);
  if (!ws || ws_bytes < need)
    return fail(W4_EWORKSPACE, "%s: workspace of %zu bytes required (got %zu)", fn, need, ws_bytes);
  if (!aligned16(ws)) return fail(W4_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  char* base = static_cast<char*>(ws);
  float* ts = tok_scale_out ? tok_scale_out : reinterpret_cast<float*>(base);
  float* tpart = ws_bytes > need ? reinterpret_cast<float*>(base + need) : nullptr;
  return launch_gemm_decomp_fused(x, M, K, N, packed, scale, zero, G, y, ts, tpart, ws_bytes - need,
                                  (hipStream_t)stream);
}

// The device address of a residual in pinned host memory (read over the host
// link) or in device memory; null for anything else (pageable memory).
static const void* residual_device_address(const uint16_t* resid) {
  hipPointerAttribute_t attr;
  const void* dev = nullptr;
  if (hipPointerGetAttributes(&attr, resid) == hipSuccess) {
    if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
      dev = resid;
    } else if (attr.type == hipMemoryTypeHost) {
      void* d = nullptr;
      if (hipHostGetDevicePointer(&d, const_cast<uint16_t*>(resid), 0) == hipSuccess) dev = d;
    }
  }
  if (!dev) (void)hipGetLastError();  // clear the query's error
  return dev;
}

int w4_salient_select(const uint16_t* x, int M, int K, int k, int32_t* idx, void* stream) {
  g_last_error[0] = '\0';
  if (M < 1 || K < 1 || K > kSelMaxK)
    return fail(W4_EINVAL, "w4_salient_select: need M >= 1 and 1 <= K <= %d (got M=%d K=%d)", kSelMaxK, M, K);
  if (k < 0 || k > K || k > kSelMaxTop)
    return fail(W4_EINVAL, "w4_salient_select: k must be in [0, min(K, %d)] (got %d)", kSelMaxTop, k);
  if (!x || (k > 0 && !idx)) return fail(W4_EINVAL, "w4_salient_select: x and idx must be non-null");
  if ((reinterpret_cast<uintptr_t>(x) & 1u) || (reinterpret_cast<uintptr_t>(idx) & 3u))
    return fail(W4_EINVAL, "w4_salient_select: x must be 2-byte and idx 4-byte aligned");
  if (k == 0) return W4_OK;
  return launch_salient_select(x, M, K, k, idx, (hipStream_t)stream);
}

int w4_residual_correct(const uint16_t* x, int M, int K, int N, const uint16_t* resid, const int32_t* idx, int k,
                        uint16_t* y, void* stream) {
  g_last_error[0] = '\0';
  if (M < 1 || M > 32 || K < 1 || N < 1 || N % 8)
    return fail(W4_EINVAL, "w4_residual_correct: need 1 <= M <= 32, K >= 1, N >= 1 with N %% 8 == 0 (got M=%d K=%d N=%d)",
                M, K, N);
  if (k < 0) return fail(W4_EINVAL, "w4_residual_correct: k must be >= 0 (got %d)", k);
  if (!x || !y || !resid || (k > 0 && !idx)) return fail(W4_EINVAL, "w4_residual_correct: null operand");
  if (!aligned16(resid) || !aligned16(y) || (reinterpret_cast<uintptr_t>(x) & 1u) ||
      (reinterpret_cast<uintptr_t>(idx) & 3u))
    return fail(W4_EINVAL, "w4_residual_correct: resid and y must be 16-byte aligned, x 2-byte, idx 4-byte");
  const void* dev = residual_device_address(resid);
  if (!dev)
    return fail(W4_EINVAL, "w4_residual_correct: resid must be pinned host memory (hipHostMalloc) or device memory");
  if (k == 0) return W4_OK;
  return launch_residual_correct(x, M, K, N, static_cast<const uint16_t*>(dev), idx, k, y, (hipStream_t)stream);
}

int w4_residual_correct_f32(const uint16_t* x, int M, int K, int N, const uint16_t* resid, const int32_t* idx,
                            int k, float* c, void* stream) {
  g_last_error[0] = '\0';
  if (M < 1 || M > 32 || K < 1 || N < 1 || N % 8)
    return fail(W4_EINVAL,
                "w4_residual_correct_f32: need 1 <= M <= 32, K >= 1, N >= 1 with N %% 8 == 0 (got M=%d K=%d N=%d)", M,
                K, N);
  if (k < 0) return fail(W4_EINVAL, "w4_residual_correct_f32: k must be >= 0 (got %d)", k);
  if (!x || !c || !resid || (k > 0 && !idx)) return fail(W4_EINVAL, "w4_residual_correct_f32: null operand");
  if (!aligned16(resid) || !aligned16(c) || (reinterpret_cast<uintptr_t>(x) & 1u) ||
      (reinterpret_cast<uintptr_t>(idx) & 3u))
    return fail(W4_EINVAL, "w4_residual_correct_f32: resid and c must be 16-byte aligned, x 2-byte, idx 4-byte");
  const void* dev = residual_device_address(resid);
  if (!dev)
    return fail(W4_EINVAL,
                "w4_residual_correct_f32: resid must be pinned host memory (hipHostMalloc) or device memory");
  return launch_residual_correct_f32(x, M, K, N, static_cast<const uint16_t*>(dev), idx, k, c, (hipStream_t)stream);
}

int w4_residual_apply(const float* c, int M, int N, uint16_t* y, void* stream) {
  g_last_error[0] = '\0';
  if (M < 1 || N < 1 || N % 8)
    return fail(W4_EINVAL, "w4_residual_apply: need M >= 1, N >= 1 with N %% 8 == 0 (got M=%d N=%d)", M, N);
  if (!c || !y) return fail(W4_EINVAL, "w4_residual_apply: null operand");
  if (!aligned16(c) || !aligned16(y)) return fail(W4_EINVAL, "w4_residual_apply: c and y must be 16-byte aligned");
  return launch_residual_apply(c, M, N, y, (hipStream_t)stream);
}

int w4_salient_correct(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k, int32_t* idx,
                       uint16_t* y, void* stream) {
  g_last_error[0] = '\0';
  if (M < 1 || M > 32 || K < 1 || K > kSelMaxK || N < 1 || N % 8)
    return fail(W4_EINVAL,
                "w4_salient_correct: need 1 <= M <= 32, 1 <= K <= %d, N >= 1 with N %% 8 == 0 (got M=%d K=%d N=%d)",
                kSelMaxK, M, K, N);
  if (k < 0 || k > K || k > kSelMaxTop)
    return fail(W4_EINVAL, "w4_salient_correct: k must be in [0, min(K, %d)] (got %d)", kSelMaxTop, k);
  if (!x || !y || !resid || (k > 0 && !idx)) return fail(W4_EINVAL, "w4_salient_correct: null operand");
  if (!aligned16(resid) || !aligned16(y) || (reinterpret_cast<uintptr_t>(x) & 1u) ||
      (reinterpret_cast<uintptr_t>(idx) & 3u))
    return fail(W4_EINVAL, "w4_salient_correct: resid and y must be 16-byte aligned, x 2-byte, idx 4-byte");
  const void* dev = residual_device_address(resid);
  if (!dev)
    return fail(W4_EINVAL, "w4_salient_correct: resid must be pinned host memory (hipHostMalloc) or device memory");
  if (k == 0) return W4_OK;
  return launch_salient_correct(x, M, K, N, static_cast<const uint16_t*>(dev), k, idx, y, (hipStream_t)stream);
}

int w4_salient_correct_f32(const uint16_t* x, int M, int K, int N, const uint16_t* resid, int k, int32_t* idx,
                           float* c, void* stream) {
  g_last_error[0] = '\0';
  if (M < 1 || M > 32 || K < 1 || K > kSelMaxK || N < 1 || N % 8)
    return fail(W4_EINVAL,
                "w4_salient_correct_f32: need 1 <= M <= 32, 1 <= K <= %d, N >= 1 with N %% 8 == 0 (got M=%d K=%d "
                "N=%d)",
                kSelMaxK, M, K, N);
  if (k < 0 || k > K || k > kSelMaxTop)
    return fail(W4_EINVAL, "w4_salient_correct_f32: k must be in [0, min(K, %d)] (got %d)", kSelMaxTop, k);
  if (!x || !c || !resid || (k > 0 && !idx)) return fail(W4_EINVAL, "w4_salient_correct_f32: null operand");
  if (!aligned16(resid) || !aligned16(c) || (reinterpret_cast<uintptr_t>(x) & 1u) ||
      (reinterpret_cast<uintptr_t>(idx) & 3u))
    return fail(W4_EINVAL, "w4_salient_correct_f32: resid and c must be 16-byte aligned, x 2-byte, idx 4-byte");
  const void* dev = residual_device_address(resid);
  if (!dev)
    return fail(W4_EINVAL,
                "w4_salient_correct_f32: resid must be pinned host memory (hipHostMalloc) or device memory");
  // k = 0: no selection (it needs k >= 1), the correction kernel writes the zeros
  if (k == 0)
    return launch_residual_correct_f32(x, M, K, N, static_cast<const uint16_t*>(dev), nullptr, 0, c,
                                       (hipStream_t)stream);
  return launch_salient_correct_f32(x, M, K, N, static_cast<const uint16_t*>(dev), k, idx, c, (hipStream_t)stream);
}

int w4_quantize_mx(const float* wt, int K, int N, uint8_t* codes, uint8_t* scale, void* stream) {
  g_last_error[0] = '\0';
  if (K < 1 || N < 1 || K % 32)
    return fail(W4_EINVAL, "w4_quantize_mx: need K, N >= 1 and K %% 32 == 0 (got K=%d N=%d)", K, N);
  if (!wt || !codes || !scale) return fail(W4_EINVAL, "w4_quantize_mx: null operand");
  if (reinterpret_cast<uintptr_t>(wt) & 3u) return fail(W4_EINVAL, "w4_quantize_mx: wt must be 4-byte aligned");
  return launch_quantize_mx(wt, K, N, codes, scale, (hipStream_t)stream);
}

int w4_pack_mx(const uint8_t* codes, int K, int N, uint8_t* packed, void* stream) {
  g_last_error[0] = '\0';
  if (K < 128 || N < 16 || K % 128 || N % 16)
    return fail(W4_EINVAL, "w4_pack_mx: need K %% 128 == 0 and N %% 16 == 0 (got K=%d N=%d)", K, N);
  if (!codes || !packed) return fail(W4_EINVAL, "w4_pack_mx: null operand");
  if (!aligned16(packed)) return fail(W4_EINVAL, "w4_pack_mx: packed must be 16-byte aligned");
  return launch_pack_mx(codes, K, N, packed, (hipStream_t)stream);
}

int w4_gemm_mx(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint8_t* scale, int nslices,
               uint16_t* y, uint8_t* slices_out, uint8_t* scales_out, void* ws, size_t ws_bytes, void* stream) {
  g_last_error[0] = '\0';
  if (M < 1 || K < 128 || N < 16 || K % 128 || N % 16)
    return fail(W4_EINVAL, "w4_gemm_mx: need M >= 1, K %% 128 == 0, N %% 16 == 0 (got M=%d K=%d N=%d)", M, K, N);
  if (nslices != 1 && nslices != 2) return fail(W4_EINVAL, "w4_gemm_mx: nslices must be 1 or 2 (got %d)", nslices);
  if (!packed || !scale) return fail(W4_EINVAL, "w4_gemm_mx: null weights");
  if (!aligned16(packed)) return fail(W4_EINVAL, "w4_gemm_mx: packed must be 16-byte aligned");
  int st;
  if ((st = check_io("w4_gemm_mx", x, y)) != W4_OK) return st;
  if (slices_out && !aligned16(slices_out)) return fail(W4_EINVAL, "w4_gemm_mx: slices_out must be 16-byte aligned");
  if ((size_t)M * (K / 2) >= (1ull << 32) || (size_t)N * (K / 2) >= (1ull << 32))
    return fail(W4_EUNSUPPORTED, "w4_gemm_mx: operands beyond the 4 GiB one call addresses");
  const size_t need = mx_workspace_bytes(M, K, nslices);
  if (!ws || ws_bytes < need)
    return fail(W4_EWORKSPACE, "w4_gemm_mx: workspace of %zu bytes required (got %zu)", need, ws_bytes);
  if (!aligned16(ws)) return fail(W4_EINVAL, "w4_gemm_mx: workspace must be 16-byte aligned");
  return launch_gemm_mx(x, M, K, N, packed, scale, nslices, y, slices_out, scales_out, ws, ws_bytes,
                        (hipStream_t)stream);
}

int w4_attn_decode_msd(const uint16_t* q, int B, int Hq, int Hkv, int L, int d, const uint8_t* k_packed,
                       const uint16_t* k_scale, const uint16_t* k_zero, const uint8_t* vt_packed,
                       const uint16_t* v_scale, const uint16_t* v_zero, uint16_t* out, void* ws, size_t ws_bytes,
                       void* stream) {
  g_last_error[0] = '\0';
  if (d != 128) return fail(W4_EUNSUPPORTED, "w4_attn_decode_msd: head dimension must be 128 (got %d)", d);
  if (B < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv || Hq / Hkv > 16)
    return fail(W4_EINVAL, "w4_attn_decode_msd: need B >= 1 and Hq a multiple of Hkv with Hq/Hkv <= 16 (got B=%d Hq=%d Hkv=%d)",
                B, Hq, Hkv);
  if (L < 256 || L % 256) return fail(W4_EINVAL, "w4_attn_decode_msd: L must be a positive multiple of 256 (got %d)", L);
  if (!q || !k_packed || !k_scale || !k_zero || !vt_packed || !v_scale || !v_zero || !out)
    return fail(W4_EINVAL, "w4_attn_decode_msd: null operand");
  if (!aligned16(q) || !aligned16(k_packed) || !aligned16(vt_packed) || (reinterpret_cast<uintptr_t>(k_scale) & 1u) ||
      (reinterpret_cast<uintptr_t>(k_zero) & 1u) || (reinterpret_cast<uintptr_t>(v_scale) & 1u) ||
      (reinterpret_cast<uintptr_t>(v_zero) & 1u) || (reinterpret_cast<uintptr_t>(out) & 1u))
    return fail(W4_EINVAL, "w4_attn_decode_msd: q and the packed caches must be 16-byte aligned, fp16 arrays 2-byte");
  const size_t need = attn_workspace_bytes(B, Hq, L);
  if (!ws || ws_bytes < need)
    return fail(W4_EWORKSPACE, "w4_attn_decode_msd: workspace of %zu bytes required (got %zu)", need, ws_bytes);
  if (!aligned16(ws)) return fail(W4_EINVAL, "w4_attn_decode_msd: workspace must be 16-byte aligned");
  return launch_attn_msd(q, B, Hq, Hkv, L, k_packed, k_scale, k_zero, vt_packed, v_scale, v_zero, out, ws,
                         (hipStream_t)stream);
}

size_t w4_workspace_bytes(int op, int M, int K, int N, int G, int fmt_or_mode) {
  switch (op) {
    case W4_OP_QUANTIZE:
    case W4_OP_PACK:
      return 0;
    case W4_OP_GEMM:
      if (M < 1 || K < 1 || N < 1 || K % 128) return 0;
      return gemm_workspace_bytes(M, K, N);
    case W4_OP_GEMV:
      if (M < 1 || M > 32 || K < 1 || N < 1 || (G != 64 && G != 128) || K % G || K % 128) return 0;
      return plan_gemv(M, K, N, G, fmt_or_mode == W4_NF4 ? W4_NF4 : W4_INT4_ASYM).ws_bytes;
    case W4_OP_ATTN_MSD:  // M = batch, K = query heads, N = positions
      if (M < 1 || K < 1 || N < 256 || N % 256) return 0;
      return attn_workspace_bytes(M, K, N);
    case W4_OP_GEMM_MX:
      if (M < 1 || K < 128 || K % 128 || (fmt_or_mode != 1 && fmt_or_mode != 2)) return 0;
      return mx_workspace_bytes(M, K, fmt_or_mode) + (N >= 16 ? mx_tail_bytes(M, K, N, fmt_or_mode) : 0);
    case W4_OP_GEMM_DECOMP:
      if (M < 1 || K < 1 || (G != 64 && G != 128) || K % G || fmt_or_mode < 1 || fmt_or_mode > 3) return 0;
      return decomp_workspace_bytes(M, K, G, fmt_or_mode) +
             (N >= 16 && K % 128 == 0 ? decomp_tail_bytes(M, K, N, G, fmt_or_mode) : 0);
    case W4_OP_GEMM_DECOMP_FUSED:
      if (M < 1 || K < 1 || (G != 64 && G != 128) || K % G) return 0;
      return decomp_fused_workspace_bytes(M) + (N >= 16 && K % 128 == 0 ? decomp_tail_bytes(M, K, N, G, 2) : 0);
    default:
      return (size_t)-1;
  }
}

int w4_stream_read(const void* buf, size_t bytes, uint32_t* xor_acc, void* stream) {
  g_last_error[0] = '\0';
  if (bytes % 16) return fail(W4_EINVAL, "w4_stream_read: bytes must be a multiple of 16 (got %zu)", bytes);
  if (bytes == 0) return W4_OK;
  if (!buf || !xor_acc) return fail(W4_EINVAL, "w4_stream_read: buf and xor_acc must be non-null");
  if (!aligned16(buf) || (reinterpret_cast<uintptr_t>(xor_acc) & 3u))
    return fail(W4_EINVAL, "w4_stream_read: buf must be 16-byte and xor_acc 4-byte aligned");
  return launch_stream_read(buf, bytes, xor_acc, (hipStream_t)stream);
}

int w4_mfma_rate(int kind, int valu, int workgroups, int iters, float* sink, unsigned long long* ticks,
                 void* stream) {
  g_last_error[0] = '\0';
  if (kind != 0 && kind != 1) return fail(W4_EINVAL, "w4_mfma_rate: kind must be 0 (fp16) or 1 (int8) (got %d)", kind);
  if (valu < 0 || valu > 8 || valu == 5 || valu == 7)
    return fail(W4_EINVAL, "w4_mfma_rate: valu must be 0, 1, 2, 3, 4, 6 or 8 (got %d)", valu);
  if (workgroups < 1 || iters < 1)
    return fail(W4_EINVAL, "w4_mfma_rate: workgroups and iters must be positive (got %d, %d)", workgroups, iters);
  if (!sink) return fail(W4_EINVAL, "w4_mfma_rate: sink must be non-null");
  if ((reinterpret_cast<uintptr_t>(sink) & 3u) || (reinterpret_cast<uintptr_t>(ticks) & 7u))
    return fail(W4_EINVAL, "w4_mfma_rate: sink must be 4-byte and ticks 8-byte aligned");
  return launch_mfma_rate(kind, valu, workgroups, iters, sink, ticks, (hipStream_t)stream);
}

int w4_nf4_levels(float* out16) {
  if (!out16) return fail(W4_EINVAL, "w4_nf4_levels: out16 must be non-null");
  std::memcpy(out16, kNf4LevelBits, sizeof(kNf4LevelBits));
  return W4_OK;
}

const char* w4_status_str(int status) {
  switch (status) {
    case W4_OK: return "W4_OK";
    case W4_EINVAL: return "W4_EINVAL: invalid argument";
    case W4_EUNSUPPORTED: return "W4_EUNSUPPORTED: unsupported request";
    case W4_EWORKSPACE: return "W4_EWORKSPACE: workspace too small";
    case W4_EHIP: return "W4_EHIP: HIP runtime error";
    default: return "unknown w4 status";
  }
}

const char* w4_last_error(void) { return g_last_error; }

const char* w4_version(void) { return "w4 0.1.0 (gfx950)"; }

}  // extern "C"

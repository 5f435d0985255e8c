// w4_gemv_noalloc: the decode GEMV for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  It runs w4_gemv's kernels and plan; the split-K
// partials that w4_gemv keeps in a caller workspace live in a fixed device
// array instead.
//
// The array, `scratch`, is a file-scope device variable: every device the
// library runs on holds its own copy until the process ends.  On the host its
// name is only a stand-in for the device symbol, so host code uses the
// address hipGetSymbolAddress returns for the current device -- looked up
// once per device, on that device's first call, with the device current --
// and passes that address to the kernels.  Calls on one device share the
// array and keep the last call's contents; the GEMV writes every partial it
// reads, so nothing needs clearing, but calls that overlap in time on one
// device race.
#include "../../include/w4.h"
#include "w4_internal.h"

#include <atomic>
#include <mutex>

namespace w4 {

// Size of the scratch (per device): room for the split-K partials of every
// GEMV plan up to this many bytes -- all the decode, MLP and decoder-layer
// shapes up to M = 32 (the largest, K = 28672, N = 8192 at M = 32, needs
// exactly this).
constexpr size_t kGemvScratchBytes = size_t(4) << 20;

static __device__ __align__(256) unsigned char scratch[kGemvScratchBytes];

namespace {

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch` (0, or a negative w4_status).
int scratch_address(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return fail(W4_EHIP, "w4_gemv_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  }
  if (dev < 0 || dev >= kScratchDevices)
    return fail(W4_EUNSUPPORTED, "w4_gemv_noalloc: device %d beyond the %d supported", dev, kScratchDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p) {
        (void)hipGetLastError();
        return fail(W4_EHIP, "w4_gemv_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      }
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return W4_OK;
}

}  // namespace
}  // namespace w4

using namespace w4;

extern "C" int w4_gemv_noalloc(const uint16_t* x, int M, int K, int N, const uint8_t* packed, const uint16_t* scale,
                               const uint16_t* zero, int G, int fmt, uint16_t* y, void* stream) {
  clear_error();
  int st;
  if ((st = check_gemv_args("w4_gemv_noalloc", x, M, K, N, packed, scale, zero, G, fmt, y)) != W4_OK) return st;
  const GemvPlan plan = plan_gemv(M, K, N, G, fmt);
  if (plan.ws_bytes > kGemvScratchBytes)
    return fail(W4_EWORKSPACE,
                "w4_gemv_noalloc: this shape needs %zu bytes of split-K partials, beyond the fixed scratch of %zu; "
                "use w4_gemv with a workspace",
                plan.ws_bytes, kGemvScratchBytes);
  void* ws = nullptr;
  if (plan.ws_bytes > 0 && (st = scratch_address(&ws)) != W4_OK) return st;
  return launch_gemv(plan, x, M, K, N, packed, scale, zero, G, fmt, y, ws, (hipStream_t)stream);
}

#include "../../include/w4.h"
#include "w4_internal.h"
namespace w4 {
int launch_gemm(const uint16_t*, int, int, int, const uint8_t*, const uint16_t*, const uint16_t*, int, int, int, uint16_t*, hipStream_t) {
  return fail(W4_EUNSUPPORTED, "w4_gemm: not built yet");
}
size_t decomp_workspace_bytes(int M, int K, int nslices) {
  return (((size_t)nslices * M * K + 255) & ~(size_t)255) + (size_t)nslices * M * sizeof(float);
}
int launch_gemm_decomp(const uint16_t*, int, int, int, const uint8_t*, const uint16_t*, const uint16_t*, int, int, uint16_t*, int8_t*, float*, int32_t*, hipStream_t) {
  return fail(W4_EUNSUPPORTED, "w4_gemm_decomp: not built yet");
}
}

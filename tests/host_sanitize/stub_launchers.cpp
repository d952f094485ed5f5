// Host-only stand-ins for the HIP launchers, for a sanitizer build of the
// C ABI's validation and dispatch (dispatch.cpp) on a machine without a GPU.
// Each launcher records which kernel the dispatcher chose and launches
// nothing.
#include "../../fp8_weight_only_fp4w_amd/csrc/launch.h"

#include <cstring>

namespace fp4w {
const char* g_last = "";
int current_device() { return 0; }
int device_cus() { return 256; }
#define STUB(name, T)          \
  int name(const T&) {         \
    g_last = #name;            \
    return 0;                  \
  }
STUB(launch_fp4_gemv, MatmulArgs)
STUB(launch_fp4_gemm, MatmulArgs)
STUB(launch_fp4_skinny, MatmulArgs)
STUB(launch_fp4_generic, MatmulArgs)
STUB(launch_fp8_gemv, MatmulArgs)
STUB(launch_fp8_gemm, MatmulArgs)
STUB(launch_fp8_skinny, MatmulArgs)
STUB(launch_fp8_generic, MatmulArgs)
STUB(launch_dequant_vec, DequantArgs)
STUB(launch_dequant_generic, DequantArgs)
STUB(launch_fp8_dequant_vec, Fp8DequantArgs)
STUB(launch_fp8_dequant_generic, Fp8DequantArgs)
STUB(launch_qdq_vec, QdqArgs)
STUB(launch_qdq_generic, QdqArgs)
#undef STUB
// what the fused W4A4 GEMV returns: 0 (launched) or 1 (A does not fit in LDS)
int g_fused_rc = 0;
int launch_fp4_gemv_w4a4(const MatmulArgs&, void*) {
  if (g_fused_rc == 0) g_last = "launch_fp4_gemv_w4a4";
  return g_fused_rc;
}
int launch_nvfp4_quantize(const Nvfp4Args&, bool vec) {
  g_last = vec ? "launch_nvfp4_quantize_vec" : "launch_nvfp4_quantize_generic";
  return 0;
}
int launch_nvfp4_qdq(const Nvfp4Args&, bool vec) {
  g_last = vec ? "launch_nvfp4_qdq_vec" : "launch_nvfp4_qdq_generic";
  return 0;
}
// a host array stands in for the device scratch (the stubs touch no memory)
int static_scratch(void** out) {
  alignas(256) static unsigned char scratch[256];
  *out = scratch;
  return 0;
}
}  // namespace fp4w

// Internal interface between the host-side dispatch (dispatch.cpp, plain C++)
// and the HIP launchers (*.hip).  Not part of the public ABI.
#pragma once

#include <stdint.h>

#include <mutex>

namespace fp4w {

enum class Act : int { F16 = 0, BF16 = 1 };

// Arguments of one matmul call after validation.  `scales` is uint8 E4M3
// bytes for FP4 and float for FP8; `ws2` is only used by FP4.
struct MatmulArgs {
  const void* A;
  const uint8_t* B;
  const void* scales;
  const float* ws2;
  const void* bias;
  void* Y;
  int64_t M, N, K, block_size, scale_cols;
  Act act;
  void* stream;  // hipStream_t
};

struct DequantArgs {
  const uint8_t* B;
  const uint8_t* scales;
  const float* ws2;
  void* out;
  int64_t N, K, block_size, scale_cols;
  Act act;
  void* stream;
};

struct Fp8DequantArgs {
  const uint8_t* B;
  const float* scales;
  void* out;
  int64_t N, K, block_size, scale_cols;
  Act act;
  void* stream;
};

// Activation quantize/dequantize (W8A8 mode): `count` elements of T.
struct QdqArgs {
  const void* A;
  const float* a_scale;
  void* out;
  int64_t count;
  Act act;
  void* stream;
};

// NVFP4 activation quantization (W4A4 path): `blocks` blocks of 16 elements
// of T.  Packed mode writes `codes` (8 bytes per block) and `scales` (1 byte
// per block); QDQ mode writes `out` (16 elements of T per block).
struct Nvfp4Args {
  const void* A;
  uint8_t* codes;
  uint8_t* scales;
  void* out;
  int64_t blocks;
  Act act;
  void* stream;
};

// Each launcher enqueues its kernel(s) and returns 0, or -1 when HIP reports
// an error at enqueue time.  Preconditions (checked by the dispatcher, never
// by the launcher) are stated next to each.

// Host-side state is per device and initialised once, thread-safely: the
// library keeps no other state between calls.
constexpr int kMaxDevices = 64;

// the calling thread's current HIP device (0 if the query fails)
int current_device();

// compute units of the current device, queried once per device (256 if the
// query fails)
int device_cus();

// Runs f() once per device for the given flag array (device ids beyond
// kMaxDevices run it on every call; f must be idempotent).
template <typename F>
void once_per_device(std::once_flag (&flags)[kMaxDevices], F&& f) {
  const int dev = current_device();
  if (dev < 0 || dev >= kMaxDevices)
    f();
  else
    std::call_once(flags[dev], f);
}

// 1 <= M <= 8, block_size == 16, K % 32 == 0, scale_cols == K / 16,
// A / B 16-byte aligned, scales 4-byte aligned, bias 2-byte aligned.
int launch_fp4_gemv(const MatmulArgs& a);
// The same GEMV with the W4A4 activation step fused: the LDS copy of A is
// NVFP4 quantize-dequantized before use and also written to a_work (M x K,
// 16-byte aligned, disjoint from A); K % 16 == 0.  Returns 1, launching
// nothing, when A does not fit in LDS or M x K / 16 exceeds 1536 blocks.
int launch_fp4_gemv_w4a4(const MatmulArgs& a, void* a_work);
// M >= 1, block_size == 16, K % 64 == 0, scale_cols == K / 16,
// A / B 16-byte aligned, scales 4-byte aligned.
int launch_fp4_gemm(const MatmulArgs& a);
// 1 <= M <= 64, block_size == 16, K % 128 == 0, scale_cols == K / 16,
// A / B 16-byte aligned, scales 4-byte aligned, bias / Y 2-byte aligned.
int launch_fp4_skinny(const MatmulArgs& a);
// any validated FP4 arguments (K may be 0)
int launch_fp4_generic(const MatmulArgs& a);

// 1 <= M <= 8, block_size % 64 == 0, K % 16 == 0, A / B 16-byte aligned,
// scales 4-byte aligned.
int launch_fp8_gemv(const MatmulArgs& a);
// M >= 1, block_size % 64 == 0, K % 64 == 0, A / B 16-byte aligned.
int launch_fp8_gemm(const MatmulArgs& a);
// 1 <= M <= 64, block_size % 128 == 0, K % 128 == 0, A / B 16-byte aligned,
// scales 4-byte aligned.
int launch_fp8_skinny(const MatmulArgs& a);
// any validated FP8 arguments (K may be 0)
int launch_fp8_generic(const MatmulArgs& a);

// K % 8 == 0, block_size % 8 == 0, B 4-byte aligned, out 16-byte aligned,
// N * K / 8 < 2^32.
int launch_dequant_vec(const DequantArgs& a);
// any validated arguments with N, K > 0
int launch_dequant_generic(const DequantArgs& a);

// FP8 dequant: K % 16 == 0, block_size % 16 == 0, B / out 16-byte aligned,
// N * K / 16 < 2^32.
int launch_fp8_dequant_vec(const Fp8DequantArgs& a);
// any validated arguments with N, K > 0
int launch_fp8_dequant_generic(const Fp8DequantArgs& a);

// count % 8 == 0, A and out 16-byte aligned; out == A allowed.
int launch_qdq_vec(const QdqArgs& a);
// any count > 0; out == A allowed.
int launch_qdq_generic(const QdqArgs& a);

// NVFP4 quantization, packed (codes and scales) or QDQ (out; out == A
// allowed).  vec: A 16-byte aligned, and codes 8-byte aligned (packed) or
// out 16-byte aligned (QDQ).  blocks > 0.
int launch_nvfp4_quantize(const Nvfp4Args& a, bool vec);
int launch_nvfp4_qdq(const Nvfp4Args& a, bool vec);

// Library-owned device scratch of the allocation-free entry point (its size
// is FP4W_STATIC_SCRATCH_BYTES of the public header): the address of the
// current device's copy, taken once per device.  0, or -1 when HIP cannot
// provide it.
constexpr int64_t kStaticScratchBytes = int64_t(32) << 20;
int static_scratch(void** out);

}  // namespace fp4w

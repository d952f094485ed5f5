// MFMA-rate probe: the dense BF16 rate the chip sustains on back-to-back,
// independent v_mfma_f32_32x32x16_bf16 instructions, the prefill GEMMs'
// instruction.  Each wave holds NACC accumulator tiles and NSET operand sets
// in registers and issues, per iteration, one MFMA per accumulator; with
// RANDOM the operand sets hold random BF16 values (random signs and
// mantissas, magnitudes 2^-4 .. 2^4) and consecutive MFMAs take different
// sets, so the operands change with every instruction as a GEMM's do; without
// it every MFMA takes the same constant operands.  The chip's clock under
// this load depends on the operand bits (switching power), so the two differ.
// A thread stores the sum of its accumulators only if its bits equal `key`,
// which the caller picks so that it never does; nothing else is written.
//
// This is measurement code, built into its own library (libmfmaprobe.so);
// the matmul library does not use it.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {  // a 32-bit integer hash (xorshift-multiply)
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// BF16 from 16 random bits: sign and 7 mantissa bits random, exponent
// 123 .. 130 (magnitudes 2^-4 .. 2^4)
__device__ __forceinline__ __bf16 random_bf16(uint32_t h) {
  const uint16_t bits = static_cast<uint16_t>((h & 0x807Fu) | ((123u + ((h >> 7) & 7u)) << 7));
  return __builtin_bit_cast(__bf16, bits);
}

template <int WAVES, int NACC, int NSET, bool RANDOM>
__global__ __launch_bounds__(256 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES, WAVES))) void mfma_peak_kernel(
    int iters, uint32_t seed, uint32_t key, float* __restrict__ sink) {
  const uint32_t tid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 a[NSET], b[NSET];
#pragma unroll
  for (int s = 0; s < NSET; ++s)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t h = RANDOM ? mix(seed ^ mix(tid * 131u + static_cast<uint32_t>(s * 8 + i))) : 0x3F80u;
      a[s][i] = RANDOM ? random_bf16(h) : __builtin_bit_cast(__bf16, static_cast<uint16_t>(0x3F80u));
      b[s][i] = RANDOM ? random_bf16(h >> 16) : __builtin_bit_cast(__bf16, static_cast<uint16_t>(0x3F00u));
    }
  f32x16 acc[NACC];
#pragma unroll
  for (int j = 0; j < NACC; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < NACC; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j % NSET], b[(j + 1) % NSET], acc[j], 0, 0, 0);
  }
  float sum = 0.0f;
#pragma unroll
  for (int j = 0; j < NACC; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[j][r];
  if (__builtin_bit_cast(uint32_t, sum) == key) sink[tid] = sum;
}

}  // namespace

// One launch of the probe on `stream`: `grid` workgroups of 256 * waves
// threads (waves = 1 or 2 per SIMD: 16 or 8 accumulator tiles per wave),
// `iters` iterations, random (1) or constant (0) operands.  sink: device
// buffer of grid * 256 * waves floats, written only where a thread's sum has
// the bits `key`.  Returns the MFMAs one launch issues (each 2 * 32 * 32 * 16
// FLOP), 0 for bad arguments (nothing launched), -1 if the launch failed.
extern "C" int64_t mfma_peak_probe(int grid, int waves, int iters, int random, uint32_t seed, uint32_t key,
                                   float* sink, hipStream_t stream) {
  if (sink == nullptr || grid < 1 || grid > 65536 || iters < 1 || (waves != 1 && waves != 2)) return 0;
  const int nacc = waves == 1 ? 16 : 8;
  const dim3 block(256 * waves);
  if (waves == 1) {
    if (random)
      hipLaunchKernelGGL((mfma_peak_kernel<1, 16, 8, true>), dim3(grid), block, 0, stream, iters, seed, key, sink);
    else
      hipLaunchKernelGGL((mfma_peak_kernel<1, 16, 8, false>), dim3(grid), block, 0, stream, iters, seed, key, sink);
  } else {
    if (random)
      hipLaunchKernelGGL((mfma_peak_kernel<2, 8, 8, true>), dim3(grid), block, 0, stream, iters, seed, key, sink);
    else
      hipLaunchKernelGGL((mfma_peak_kernel<2, 8, 8, false>), dim3(grid), block, 0, stream, iters, seed, key, sink);
  }
  if (hipGetLastError() != hipSuccess) return -1;
  return static_cast<int64_t>(grid) * 4 * waves * iters * nacc;
}

// FP4 and FP8 -> FP16/BF16 dequant kernels (the library's fp4w_dequant and
// fp8w_dequant).
//
// out[n, k] = RNE_T( RNE_f32( e2m1(B[n,k]) * e4m3(ws[n, col(k)]) * ws2 ) )
// ([FP4 doc] §2 Weight Format; [FP4 doc] §5 step 1; the vectorised kernel of
// [Blog], sections "The new kernel assigns eight FP4 values to each thread"
// through "The tensor-level scale is loaded once and reused").
//
// What differs from the pages' CUDA kernel, for gfx950:
//  * one flat grid-stride loop over 8-element chunks, with row and column
//    recovered by multiply-high division (constants computed on the host)
//    instead of a 2-D grid: the output is one contiguous [N*K] stream, so
//    every wave64 store instruction writes 1 KiB of consecutive bytes and
//    N = 152064 rows need no y-grid-limit handling;
//  * decode through v_cvt_scalef32_pk_f32_fp4 (E2M1 pair -> FP32, exact) and
//    v_cvt_f32_fp8 (E4M3 -> FP32, exact), then two FP32 multiplies in the
//    order of the formula, then one rounding to T;
//  * the tensor scale ws2 is one scalar load per thread, kept in a register.
//
// FP8: out[n, k] = RNE_T( RNE_f32( e4m3(B[n, k]) * b_scale[n, col(k)] ) ),
// the expansion of the FP8 operator's default path ([FP8 doc] §5, step 1,
// whose fast kernel gives each thread one aligned 16-element K chunk).  Here
// too a 16-element chunk (one 16-byte load, two 16-byte stores) stays inside
// one scale block when block_size % 16 == 0, so one FP32 scale is read per
// chunk; the chunks form one flat grid-stride stream as for FP4.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"
// [Blog]    = "ONNX Runtime #32128 - Why Dequantizing 4-Bit Weights Became the
//             Most Expensive Kernel in H200 Prefill"

#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

template <typename T>
struct Store8;
template <>
struct Store8<__bf16> {
  __device__ __forceinline__ static u32x4 pack(const float (&v)[8]) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = round_to<__bf16>(v[i]);
    return __builtin_bit_cast(u32x4, r);
  }
};
template <>
struct Store8<_Float16> {
  __device__ __forceinline__ static u32x4 pack(const float (&v)[8]) {
    f16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = round_to<_Float16>(v[i]);
    return __builtin_bit_cast(u32x4, r);
  }
};

constexpr int kDqThreads = 256;
constexpr int kDqUnroll = 4;  // chunks in flight per thread

// One chunk = 8 consecutive k of one row = one 32-bit packed word and one
// 16-byte output vector; every chunk lies inside one scale block because
// block_size % 8 == 0.
template <typename T>
__global__ __launch_bounds__(kDqThreads) void dequant_vec_kernel(
    const uint32_t* __restrict__ Bw, const uint8_t* __restrict__ ws, const float* __restrict__ ws2p,
    u32x4* __restrict__ out, uint32_t total_chunks, FastDiv chunks_per_row, FastDiv chunks_per_block,
    uint32_t cols) {
  const float ws2 = *ws2p;
  const uint32_t stride = gridDim.x * kDqThreads * kDqUnroll;
  for (uint32_t base = blockIdx.x * kDqThreads * kDqUnroll + threadIdx.x; base < total_chunks;
       base += stride) {
    uint32_t word[kDqUnroll];
    uint32_t sbyte[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const uint32_t c = base + u * kDqThreads;
      if (c < total_chunks) {
        const uint32_t row = fdiv(c, chunks_per_row);
        const uint32_t cc = c - row * chunks_per_row.d;
        const uint32_t col = min(fdiv(cc, chunks_per_block), cols - 1);
        word[u] = Bw[c];
        sbyte[u] = ws[static_cast<uint64_t>(row) * cols + col];
      }
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const uint32_t c = base + u * kDqThreads;
      if (c < total_chunks) {
        const float s = e4m3_to_f32<0>(sbyte[u]);
        const f32x2 q0 = e2m1x2_to_f32<0>(word[u]);
        const f32x2 q1 = e2m1x2_to_f32<1>(word[u]);
        const f32x2 q2 = e2m1x2_to_f32<2>(word[u]);
        const f32x2 q3 = e2m1x2_to_f32<3>(word[u]);
        // (e2m1 * e4m3) is exact; the multiply by ws2 is the one FP32 rounding
        float v[8] = {(q0.x * s) * ws2, (q0.y * s) * ws2, (q1.x * s) * ws2, (q1.y * s) * ws2,
                      (q2.x * s) * ws2, (q2.y * s) * ws2, (q3.x * s) * ws2, (q3.y * s) * ws2};
        out[c] = Store8<T>::pack(v);
      }
    }
  }
}

// Any shape: one element per iteration, scale column per element (odd
// block_size may split a packed byte between two scale blocks: [Blog], "Why
// the block size must be even").
template <typename T>
__global__ __launch_bounds__(256) void dequant_generic_kernel(
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ ws, const float* __restrict__ ws2p,
    T* __restrict__ out, int64_t N, int64_t K, int64_t bs, int64_t cols) {
  const float ws2 = *ws2p;
  const int64_t total = N * K;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = e / K;
    const int64_t k = e - row * K;
    const uint32_t byte = B[row * (K / 2) + (k >> 1)];
    const f32x2 q2 = e2m1x2_to_f32<0>(byte);
    const float q = (k & 1) ? q2.y : q2.x;
    const int64_t col = min(k / bs, cols - 1);
    const float s = e4m3_to_f32<0>(ws[row * cols + col]);
    out[e] = round_to<T>((q * s) * ws2);
  }
}

// FP8, 16 elements per chunk: one 16-byte weight load, one scale, two
// 16-byte stores.
template <typename T>
__global__ __launch_bounds__(kDqThreads) void fp8_dequant_vec_kernel(
    const u32x4* __restrict__ Bv, const float* __restrict__ scales, u32x4* __restrict__ out,
    uint32_t total_chunks, FastDiv chunks_per_row, FastDiv chunks_per_block, uint32_t cols) {
  const uint32_t stride = gridDim.x * kDqThreads * kDqUnroll;
  for (uint32_t base = blockIdx.x * kDqThreads * kDqUnroll + threadIdx.x; base < total_chunks;
       base += stride) {
    u32x4 w[kDqUnroll];
    float sc[kDqUnroll];
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const uint32_t c = base + u * kDqThreads;
      if (c < total_chunks) {
        const uint32_t row = fdiv(c, chunks_per_row);
        const uint32_t cc = c - row * chunks_per_row.d;
        const uint32_t col = min(fdiv(cc, chunks_per_block), cols - 1);
        w[u] = Bv[c];
        sc[u] = scales[static_cast<uint64_t>(row) * cols + col];
      }
    }
#pragma unroll
    for (int u = 0; u < kDqUnroll; ++u) {
      const uint32_t c = base + u * kDqThreads;
      if (c < total_chunks) {
        out[2 * static_cast<uint64_t>(c)] = __builtin_bit_cast(u32x4, decode8_fp8_scaled<T>(w[u].x, w[u].y, sc[u]));
        out[2 * static_cast<uint64_t>(c) + 1] =
            __builtin_bit_cast(u32x4, decode8_fp8_scaled<T>(w[u].z, w[u].w, sc[u]));
      }
    }
  }
}

// FP8, any shape: one element per iteration.
template <typename T>
__global__ __launch_bounds__(256) void fp8_dequant_generic_kernel(
    const uint8_t* __restrict__ B, const float* __restrict__ scales, T* __restrict__ out, int64_t N,
    int64_t K, int64_t bs, int64_t cols) {
  const int64_t total = N * K;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
       e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = e / K;
    const int64_t k = e - row * K;
    const float q = e4m3_to_f32<0>(B[e]);
    const float s = scales[row * cols + min(k / bs, cols - 1)];
    out[e] = round_to<T>(q * s);
  }
}

int grid_for(int64_t work_items, int per_block) {
  int64_t g = (work_items + per_block - 1) / per_block;
  const int64_t cap = 256 * 16;  // 256 CUs, enough waves in flight to cover HBM latency
  if (g > cap) g = cap;
  if (g < 1) g = 1;
  return static_cast<int>(g);
}

}  // namespace

int launch_dequant_vec(const DequantArgs& a) {
  const uint32_t cpr = static_cast<uint32_t>(a.K / 8);
  const uint32_t total = static_cast<uint32_t>(a.N * (a.K / 8));
  const FastDiv f_row = make_fastdiv(cpr);
  const FastDiv f_blk = make_fastdiv(static_cast<uint32_t>(a.block_size / 8));
  const int grid = grid_for(total, kDqThreads * kDqUnroll);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  if (a.act == Act::BF16)
    hipLaunchKernelGGL(dequant_vec_kernel<__bf16>, dim3(grid), dim3(kDqThreads), 0, s,
                       reinterpret_cast<const uint32_t*>(a.B), a.scales, a.ws2,
                       static_cast<u32x4*>(a.out), total, f_row, f_blk,
                       static_cast<uint32_t>(a.scale_cols));
  else
    hipLaunchKernelGGL(dequant_vec_kernel<_Float16>, dim3(grid), dim3(kDqThreads), 0, s,
                       reinterpret_cast<const uint32_t*>(a.B), a.scales, a.ws2,
                       static_cast<u32x4*>(a.out), total, f_row, f_blk,
                       static_cast<uint32_t>(a.scale_cols));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_dequant_generic(const DequantArgs& a) {
  const int grid = grid_for(a.N * a.K, 256);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  if (a.act == Act::BF16)
    hipLaunchKernelGGL(dequant_generic_kernel<__bf16>, dim3(grid), dim3(256), 0, s, a.B, a.scales,
                       a.ws2, static_cast<__bf16*>(a.out), a.N, a.K, a.block_size, a.scale_cols);
  else
    hipLaunchKernelGGL(dequant_generic_kernel<_Float16>, dim3(grid), dim3(256), 0, s, a.B, a.scales,
                       a.ws2, static_cast<_Float16*>(a.out), a.N, a.K, a.block_size, a.scale_cols);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fp8_dequant_vec(const Fp8DequantArgs& a) {
  const uint32_t cpr = static_cast<uint32_t>(a.K / 16);
  const uint32_t total = static_cast<uint32_t>(a.N * (a.K / 16));
  const FastDiv f_row = make_fastdiv(cpr);
  const FastDiv f_blk = make_fastdiv(static_cast<uint32_t>(a.block_size / 16));
  const int grid = grid_for(total, kDqThreads * kDqUnroll);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  if (a.act == Act::BF16)
    hipLaunchKernelGGL(fp8_dequant_vec_kernel<__bf16>, dim3(grid), dim3(kDqThreads), 0, s,
                       reinterpret_cast<const u32x4*>(a.B), a.scales, static_cast<u32x4*>(a.out), total,
                       f_row, f_blk, static_cast<uint32_t>(a.scale_cols));
  else
    hipLaunchKernelGGL(fp8_dequant_vec_kernel<_Float16>, dim3(grid), dim3(kDqThreads), 0, s,
                       reinterpret_cast<const u32x4*>(a.B), a.scales, static_cast<u32x4*>(a.out), total,
                       f_row, f_blk, static_cast<uint32_t>(a.scale_cols));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fp8_dequant_generic(const Fp8DequantArgs& a) {
  const int grid = grid_for(a.N * a.K, 256);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
  if (a.act == Act::BF16)
    hipLaunchKernelGGL(fp8_dequant_generic_kernel<__bf16>, dim3(grid), dim3(256), 0, s, a.B, a.scales,
                       static_cast<__bf16*>(a.out), a.N, a.K, a.block_size, a.scale_cols);
  else
    hipLaunchKernelGGL(fp8_dequant_generic_kernel<_Float16>, dim3(grid), dim3(256), 0, s, a.B, a.scales,
                       static_cast<_Float16*>(a.out), a.N, a.K, a.block_size, a.scale_cols);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fp4w

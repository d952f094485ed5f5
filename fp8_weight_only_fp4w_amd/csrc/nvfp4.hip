// NVFP4 activation quantization, step 1 of the FP4 operator's native
// FP4 x FP4 path ([FP4 doc] §6 Native SM120 FP4 x FP4 Path): each block of 16
// consecutive elements of a row of A becomes 16 E2M1 codes and one E4M3
// scale.  The pages name the format only; the rules used here (stated with
// the public entry points) are:
//
//   scale = e4m3( sat448( RNE_f32(amax / 6) ) )      NaN in the block -> NaN
//   code  = e2m1( RNE_f32(a / scale) )                scale 0 -> code 0
//
// with e4m3 and e2m1 the nearest value, ties to the even code, e2m1
// saturating at 6 and keeping the sign.  Both quotients are IEEE FP32
// divisions (the second one is decided without dividing, below).  The QDQ
// form writes e2m1 x e4m3 back in T, which is exact (at most 6 significand
// bits, magnitudes within [2^-10, 2688]): a W4A4 matmul is that activation
// times the dequantized weights, run by the FP4 GEMM.
//
// gfx950 mapping: one thread per block (32 bytes of T in, 9 bytes or 32 bytes
// out, contiguous across the wave), a flat grid-stride loop; v_cvt_pk_fp8_f32
// encodes the scale (round to nearest even), v_cvt_f32_fp8 and
// v_cvt_scalef32_pk_f32_fp4 decode scale and codes exactly.
//
// The element code needs no division.  The E2M1 rounding boundaries of a / s
// are the midpoints t in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}; t * s is
// exact in FP32 (at most 3 + 4 significand bits), so |a| against t * s
// decides the exact quotient's side of each boundary, ties included.  The
// rounded quotient RNE_f32(a / s) falls on the same side: a (at most 11
// significand bits for FP16, 8 for BF16; t * s is at least 2^-11) either
// equals t * s or differs from it by at least 2^-13 of its size, far more
// than half an FP32 ulp, so rounding the quotient never moves it onto or
// across a boundary.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"

#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr int kThreads = 256;

// E2M1 code of a / s from the boundaries t * s (thr, see above): the
// magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 and their midpoints, each tie going
// to the neighbour with the even code; saturating at 6; the sign of a kept
__device__ __forceinline__ uint32_t e2m1_code(float a, const float (&thr)[7]) {
  const float m = fabsf(a);
  const uint32_t c = (m > thr[0]) + (m >= thr[1]) + (m > thr[2]) + (m >= thr[3]) + (m > thr[4]) +
                     (m >= thr[5]) + (m > thr[6]);
  return c | ((__float_as_uint(a) >> 28) & 8u);
}

// one block: its 16 values -> scale byte, decoded scale and two words of
// codes (element i in bits 4 (i % 8) of word i / 8)
__device__ __forceinline__ void quant_block(const float (&v)[16], uint32_t& sbyte, float& s, uint32_t (&w)[2]) {
  float amax = 0.0f;
  bool nan = false;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    nan |= v[i] != v[i];
    amax = fmaxf(amax, fabsf(v[i]));
  }
  if (nan) {
    sbyte = 0x7Fu;
    s = __builtin_nanf("");
  } else {
    float r = amax / 6.0f;
    r = r > 448.0f ? 448.0f : r;  // E4M3 "fn" has no infinity: saturate
    sbyte = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.0f, 0, false)) & 0xFFu;
    s = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(sbyte), 0);
  }
  w[0] = 0u;
  w[1] = 0u;
  if (s > 0.0f) {  // a zero or NaN scale leaves every code 0
    const float thr[7] = {0.25f * s, 0.75f * s, 1.25f * s, 1.75f * s, 2.5f * s, 3.5f * s, 5.0f * s};
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i >> 3] |= e2m1_code(v[i], thr) << (4 * (i & 7));
  }
}

template <typename T, bool VEC>
__device__ __forceinline__ void load_block(const T* A, int64_t b, float (&v)[16]) {
  if constexpr (VEC) {
    typedef typename ActTraits<T>::vec8 V;
    const u32x4* p = reinterpret_cast<const u32x4*>(A + 16 * b);
    const V x0 = __builtin_bit_cast(V, p[0]);
    const V x1 = __builtin_bit_cast(V, p[1]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[i] = static_cast<float>(x0[i]);
      v[8 + i] = static_cast<float>(x1[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = static_cast<float>(A[16 * b + i]);
  }
}

template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void nvfp4_quantize_kernel(const T* A, uint8_t* codes, uint8_t* scales,
                                                                  int64_t blocks) {
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < blocks;
       b += static_cast<int64_t>(gridDim.x) * kThreads) {
    float v[16];
    load_block<T, VEC>(A, b, v);
    uint32_t sbyte, w[2];
    float s;
    quant_block(v, sbyte, s, w);
    if constexpr (VEC) {
      *reinterpret_cast<u32x2*>(codes + 8 * b) = u32x2{w[0], w[1]};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) codes[8 * b + i] = static_cast<uint8_t>(w[i >> 2] >> (8 * (i & 3)));
    }
    scales[b] = static_cast<uint8_t>(sbyte);
  }
}

// In-place use (out == A) is safe: every block is read and written by the
// same thread, the read first (hence no __restrict__).
template <typename T, bool VEC>
__global__ __launch_bounds__(kThreads) void nvfp4_qdq_kernel(const T* A, T* out, int64_t blocks) {
  typedef typename ActTraits<T>::vec8 V;
  for (int64_t b = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; b < blocks;
       b += static_cast<int64_t>(gridDim.x) * kThreads) {
    float v[16];
    load_block<T, VEC>(A, b, v);
    uint32_t sbyte, w[2];
    float s;
    quant_block(v, sbyte, s, w);
    // decode: e2m1 x e4m3 is exact in FP32 and in T
    V r[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const f32x2 p0 = e2m1x2_to_f32<0>(w[h]), p1 = e2m1x2_to_f32<1>(w[h]);
      const f32x2 p2 = e2m1x2_to_f32<2>(w[h]), p3 = e2m1x2_to_f32<3>(w[h]);
      r[h][0] = round_to<T>(p0.x * s); r[h][1] = round_to<T>(p0.y * s);
      r[h][2] = round_to<T>(p1.x * s); r[h][3] = round_to<T>(p1.y * s);
      r[h][4] = round_to<T>(p2.x * s); r[h][5] = round_to<T>(p2.y * s);
      r[h][6] = round_to<T>(p3.x * s); r[h][7] = round_to<T>(p3.y * s);
    }
    if constexpr (VEC) {
      u32x4* q = reinterpret_cast<u32x4*>(out + 16 * b);
      q[0] = __builtin_bit_cast(u32x4, r[0]);
      q[1] = __builtin_bit_cast(u32x4, r[1]);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) out[16 * b + i] = r[i >> 3][i & 7];
    }
  }
}

int grid_for(int64_t blocks) {
  int64_t g = (blocks + kThreads - 1) / kThreads;
  const int64_t cap = 256 * 16;
  return static_cast<int>(g > cap ? cap : (g < 1 ? 1 : g));
}

template <typename T>
int quantize_t(const Nvfp4Args& a, bool vec) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const T* A = static_cast<const T*>(a.A);
  if (vec)
    hipLaunchKernelGGL((nvfp4_quantize_kernel<T, true>), dim3(grid_for(a.blocks)), dim3(kThreads), 0, st, A,
                       a.codes, a.scales, a.blocks);
  else
    hipLaunchKernelGGL((nvfp4_quantize_kernel<T, false>), dim3(grid_for(a.blocks)), dim3(kThreads), 0, st, A,
                       a.codes, a.scales, a.blocks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

template <typename T>
int qdq_t(const Nvfp4Args& a, bool vec) {
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const T* A = static_cast<const T*>(a.A);
  T* out = static_cast<T*>(a.out);
  if (vec)
    hipLaunchKernelGGL((nvfp4_qdq_kernel<T, true>), dim3(grid_for(a.blocks)), dim3(kThreads), 0, st, A, out,
                       a.blocks);
  else
    hipLaunchKernelGGL((nvfp4_qdq_kernel<T, false>), dim3(grid_for(a.blocks)), dim3(kThreads), 0, st, A, out,
                       a.blocks);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_nvfp4_quantize(const Nvfp4Args& a, bool vec) {
  return a.act == Act::BF16 ? quantize_t<__bf16>(a, vec) : quantize_t<_Float16>(a, vec);
}

int launch_nvfp4_qdq(const Nvfp4Args& a, bool vec) {
  return a.act == Act::BF16 ? qdq_t<__bf16>(a, vec) : qdq_t<_Float16>(a, vec);
}

}  // namespace fp4w

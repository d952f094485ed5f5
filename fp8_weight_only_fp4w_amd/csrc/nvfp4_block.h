// NVFP4 quantization of one block of 16 activations, shared by the
// standalone activation kernels (nvfp4.hip) and the decode GEMV's W4A4 mode
// (gemv.hip), so that both produce the same codes and scales.  The rules
// ([FP4 doc] §6 names the format only) are:
//
//   scale = e4m3( sat448( RNE_f32(amax / 6) ) )      NaN in the block -> NaN
//   code  = e2m1( RNE_f32(a / scale) )                scale 0 -> code 0
//
// with e4m3 and e2m1 the nearest value, ties to the even code, e2m1
// saturating at 6 and keeping the sign.  Both quotients are IEEE FP32
// divisions (the second one is decided without dividing, below).
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
#pragma once

#include "device.h"

namespace fp4w {

// E2M1 code of a / s from the boundaries t * s (thr, see above): the
// magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 and their midpoints, each tie going
// to the neighbour with the even code; saturating at 6; the sign of a kept
__device__ __forceinline__ uint32_t nvfp4_e2m1_code(float a, const float (&thr)[7]) {
  const float m = fabsf(a);
  const uint32_t c = (m > thr[0]) + (m >= thr[1]) + (m > thr[2]) + (m >= thr[3]) + (m > thr[4]) +
                     (m >= thr[5]) + (m > thr[6]);
  return c | ((__float_as_uint(a) >> 28) & 8u);
}

// one block: its 16 values -> scale byte, decoded scale and two words of
// codes (element i in bits 4 (i % 8) of word i / 8)
__device__ __forceinline__ void nvfp4_quant_block(const float (&v)[16], uint32_t& sbyte, float& s,
                                                  uint32_t (&w)[2]) {
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
    for (int i = 0; i < 16; ++i) w[i >> 3] |= nvfp4_e2m1_code(v[i], thr) << (4 * (i & 7));
  }
}

// One block quantized and dequantized, without forming the codes.  The
// value is sign(a) * e2m1(q) * s, q = |a| / s, and e2m1(q) is reached in
// float arithmetic:
//   * q' = |a| * rcp(s) is within 2^-22 of q (relative).  Rounding q' to 20
//     significant bits gives every tie (q equal to a boundary t, at most 3
//     significant bits) exactly, and moves no other quotient onto or across
//     a boundary: those are at least 2^-13 (relative) away from every t (see
//     above), far beyond the 2^-20 the two steps can move them.
//   * adding and subtracting c = 2^(22 + floor(log2 clamp(q, 1, 8))) rounds q
//     to the E2M1 step of its binade (0.5 below 2, then 1, then 2), ties to
//     even, which is the E2M1 rounding: each tie goes to the even code;
//     anything from 7 up reaches 8 or more, which saturates to 6.
// e2m1 x e4m3 is exact in FP32 and in T (at most 6 significand bits,
// magnitudes within [2^-10, 2688]).  A block with a zero scale (or NaN)
// gives +0 (NaN) everywhere, as its codes are all 0.
template <typename T>
__device__ __forceinline__ void nvfp4_qdq_block(const float (&v)[16], typename ActTraits<T>::vec8 (&r)[2]) {
  uint32_t mx = 0u;  // largest magnitude, as bits: above +inf's means a NaN
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = max(mx, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  float s;
  if (mx > 0x7F800000u) {
    s = __builtin_nanf("");
  } else {
    float q = __uint_as_float(mx) / 6.0f;
    q = q > 448.0f ? 448.0f : q;
    s = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(__builtin_amdgcn_cvt_pk_fp8_f32(q, 0.0f, 0, false) & 0xFF), 0);
  }
  const bool live = s > 0.0f;
  const float inv = live ? __builtin_amdgcn_rcpf(s) : 0.0f;
  const uint32_t sign_mask = live ? 0x80000000u : 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float q = fabsf(v[i]) * inv;
    q = __uint_as_float((__float_as_uint(q) + 8u) & ~15u);
    const float c = __uint_as_float((__float_as_uint(__builtin_amdgcn_fmed3f(q, 1.0f, 8.0f)) & 0x7F800000u) +
                                    (22u << 23));
    const float e = fminf(f32_barrier(f32_barrier(q + c) - c), 6.0f);
    const float o = __uint_as_float(__float_as_uint(e * s) | (__float_as_uint(v[i]) & sign_mask));
    r[i >> 3][i & 7] = round_to<T>(o);
  }
}

}  // namespace fp4w

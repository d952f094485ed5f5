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
// The element code needs no division: the E2M1 rounding boundaries of a / s
// are the midpoints t in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}, and the
// rounded quotient RNE_f32(a / s) falls on the same side of each as the
// exact one: a (at most 11 significand bits for FP16, 8 for BF16; t * s,
// exact in FP32, is at least 2^-11) either equals t * s or differs from it
// by at least 2^-13 of its size, far more than half an FP32 ulp.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
#pragma once

#include "device.h"

namespace fp4w {

// The block's scale: its byte and FP32 value, NaN for a block with a NaN
// (the largest magnitude, taken on the bits, is then above +inf's).
__device__ __forceinline__ void nvfp4_block_scale(const float (&v)[16], uint32_t& sbyte, float& s) {
  uint32_t mx = 0u;
#pragma unroll
  for (int i = 0; i < 16; ++i) mx = max(mx, __float_as_uint(v[i]) & 0x7FFFFFFFu);
  if (mx > 0x7F800000u) {
    sbyte = 0x7Fu;
    s = __builtin_nanf("");
  } else {
    float r = __uint_as_float(mx) / 6.0f;
    r = r > 448.0f ? 448.0f : r;  // E4M3 "fn" has no infinity: saturate
    sbyte = static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(r, 0.0f, 0, false)) & 0xFFu;
    s = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(sbyte), 0);
  }
}

// The block's 16 codes (element i in bits 4 (i % 8) of word i / 8), without
// a division.  q' = a * rcp(s) is within 2^-22 of a / s (relative); rounded
// to 20 significant bits (magnitude, half away from zero) it equals every
// tie exactly (a boundary t of the E2M1 grid has at most 3 significant bits)
// and stays on the same side of every boundary as a / s otherwise (those
// quotients lie at least 2^-13 from every t, see above; the two roundings
// move them by at most 2^-20).  v_cvt_scalef32_pk_fp4_f32 with scale 1 then
// rounds it to the E2M1 grid: nearest, ties to the even code, saturating at
// 6, the sign kept (also on a zero); the GPU tests check this on every FP16
// and BF16 pattern.  A zero or NaN scale leaves every code 0.
__device__ __forceinline__ void nvfp4_block_codes(const float (&v)[16], float s, uint32_t (&w)[2]) {
  const bool live = s > 0.0f;
  const float inv = __builtin_amdgcn_rcpf(s);
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) q[i] = __uint_as_float((__float_as_uint(v[i] * inv) + 8u) & ~15u);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t x = 0u;
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[8 * h + 0], q[8 * h + 1], 1.0f, 0);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[8 * h + 2], q[8 * h + 3], 1.0f, 1);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[8 * h + 4], q[8 * h + 5], 1.0f, 2);
    x = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(x, q[8 * h + 6], q[8 * h + 7], 1.0f, 3);
    w[h] = live ? x : 0u;
  }
}

// one block: its 16 values -> scale byte, decoded scale and two words of
// codes (element i in bits 4 (i % 8) of word i / 8)
__device__ __forceinline__ void nvfp4_quant_block(const float (&v)[16], uint32_t& sbyte, float& s,
                                                  uint32_t (&w)[2]) {
  nvfp4_block_scale(v, sbyte, s);
  nvfp4_block_codes(v, s, w);
}

// one block quantized and dequantized: e2m1 x e4m3 is exact in FP32 and in
// T (at most 6 significand bits, magnitudes within [2^-10, 2688]); a block
// with a zero (NaN) scale gives +0 (NaN) everywhere
template <typename T>
__device__ __forceinline__ void nvfp4_qdq_block(const float (&v)[16], typename ActTraits<T>::vec8 (&r)[2]) {
  uint32_t sbyte, w[2];
  float s;
  nvfp4_quant_block(v, sbyte, s, w);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x2 p0 = e2m1x2_to_f32<0>(w[h]), p1 = e2m1x2_to_f32<1>(w[h]);
    const f32x2 p2 = e2m1x2_to_f32<2>(w[h]), p3 = e2m1x2_to_f32<3>(w[h]);
    r[h][0] = round_to<T>(p0.x * s); r[h][1] = round_to<T>(p0.y * s);
    r[h][2] = round_to<T>(p1.x * s); r[h][3] = round_to<T>(p1.y * s);
    r[h][4] = round_to<T>(p2.x * s); r[h][5] = round_to<T>(p2.y * s);
    r[h][6] = round_to<T>(p3.x * s); r[h][7] = round_to<T>(p3.y * s);
  }
}

}  // namespace fp4w

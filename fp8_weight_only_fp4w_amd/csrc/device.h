// Device helpers shared by the gfx950 kernels: vector types, E2M1 / E4M3
// decode through the CDNA4 conversion instructions, and output rounding.
//
// Facts these helpers rely on (each checked on gfx950 over every input code):
//  * v_cvt_f32_fp8 / v_cvt_pk_f32_fp8 / v_cvt_scalef32_pk_{f16,bf16}_fp8 with
//    scale 1.0 decode the OCP E4M3 "fn" format (bias 7, max 448, NaN only at
//    0x7F / 0xFF), the weight and scale format of the pages ([FP4 doc] §2,
//    [FP8 doc] §1).
//  * v_cvt_scalef32_pk_{f32,f16,bf16}_fp4 with scale 1.0 decode E2M1 exactly,
//    -0.0 included.  The scale operand contributes only its power of two, so
//    the E4M3 block scale (4 significand bits) is applied with a separate
//    multiply, never through that operand.
//  * FP32 and FP16 denormals are kept (no flush to zero) and FP32 -> FP16 /
//    BF16 conversions round to nearest even.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4w {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ------------------------------------------------------------------ E4M3

// E4M3 byte `SEL` (0..3) of `word` -> FP32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(word), SEL);
}

// ------------------------------------------------------------------ E2M1

// E2M1 pair in byte `SEL` of `word` -> two FP32 values (exact; .x = low nibble).
template <int SEL>
__device__ __forceinline__ f32x2 e2m1x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// ------------------------------------------------------------------ operand build

// Activation-type traits: how an 8-wide MFMA operand of T is formed from the
// E2M1 codes of one 32-bit word (8 codes, low nibble first) times a block
// scale.  E2M1 x E4M3 needs at most 6 significand bits and lies in
// [2^-10, 2688], so the product is exact in FP16 and in BF16 ([FP4 doc] §4,
// tensor-core sub-path): folding the scale into the operand loses nothing.
template <typename T>
struct ActTraits;

template <>
struct ActTraits<__bf16> {
  typedef bf16x8 vec8;
  typedef float scale_t;  // FP32 copy of the E4M3 scale
  __device__ __forceinline__ static scale_t make_scale(float s) { return s; }
  __device__ __forceinline__ static bf16x2 pack(float a, float b) {
    bf16x2 r;
    r[0] = static_cast<__bf16>(a);
    r[1] = static_cast<__bf16>(b);
    return r;
  }
  // 8 E2M1 codes of `w` times s -> bf16x8 (exact)
  __device__ __forceinline__ static vec8 decode8(uint32_t w, scale_t s) {
    f32x2 p0 = e2m1x2_to_f32<0>(w) * s;
    f32x2 p1 = e2m1x2_to_f32<1>(w) * s;
    f32x2 p2 = e2m1x2_to_f32<2>(w) * s;
    f32x2 p3 = e2m1x2_to_f32<3>(w) * s;
    vec8 r;
    r[0] = static_cast<__bf16>(p0.x); r[1] = static_cast<__bf16>(p0.y);
    r[2] = static_cast<__bf16>(p1.x); r[3] = static_cast<__bf16>(p1.y);
    r[4] = static_cast<__bf16>(p2.x); r[5] = static_cast<__bf16>(p2.y);
    r[6] = static_cast<__bf16>(p3.x); r[7] = static_cast<__bf16>(p3.y);
    return r;
  }
  // 8 E2M1 codes of `w` -> bf16x8 (exact, no scale)
  __device__ __forceinline__ static vec8 decode8_fp4(uint32_t w) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    vec8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
  }
  // 8 E4M3 codes of (lo, hi) -> bf16x8 (exact, no scale)
  __device__ __forceinline__ static vec8 decode8_fp8(uint32_t lo, uint32_t hi) {
    bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
    bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
    bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
    bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
    vec8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
  }
  __device__ __forceinline__ static f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static float to_f32(__bf16 x) { return static_cast<float>(x); }
};

template <>
struct ActTraits<_Float16> {
  typedef f16x8 vec8;
  typedef f16x2 scale_t;  // (s, s) in FP16: every E4M3 value is exact in FP16
  __device__ __forceinline__ static scale_t make_scale(float s) {
    f16x2 r;
    r[0] = static_cast<_Float16>(s);
    r[1] = r[0];
    return r;
  }
  __device__ __forceinline__ static vec8 decode8(uint32_t w, scale_t s) {
    f16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
    f16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
    f16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
    f16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
    vec8 r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
  }
  __device__ __forceinline__ static vec8 decode8_fp4(uint32_t w) {
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
    vec8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
  }
  __device__ __forceinline__ static vec8 decode8_fp8(uint32_t lo, uint32_t hi) {
    f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
    f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
    f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
    f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
    vec8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
    r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
    return r;
  }
  __device__ __forceinline__ static f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static float to_f32(_Float16 x) { return static_cast<float>(x); }
};

// Materialise an FP32 value in a VGPR.  Without this the backend may fold
// "multiply in FP32, then convert to FP16" into one mixed-precision FMA
// (v_fma_mix*_f16 with a +0 addend), which rounds once instead of twice and
// turns -0 into +0.  The stored result is defined as RNE_T(RNE_f32(.)), so
// every FP32 -> T output conversion goes through this barrier (it emits no
// instruction).
__device__ __forceinline__ float f32_barrier(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// FP32 -> T, round to nearest even, from an FP32 value that has been rounded.
template <typename T>
__device__ __forceinline__ T round_to(float x) {
  return static_cast<T>(f32_barrier(x));
}

// 8 E4M3 codes of (lo, hi), low byte first, times an FP32 scale -> 8 x T:
// each product is rounded once to FP32 and once to T, the dequantized weight
// in the activation type (exact for the E4M3 code, rounded for the scale).
template <typename T>
__device__ __forceinline__ typename ActTraits<T>::vec8 decode8_fp8_scaled(uint32_t lo, uint32_t hi, float s) {
  const f32x2 p0 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(lo), false);
  const f32x2 p1 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(lo), true);
  const f32x2 p2 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(hi), false);
  const f32x2 p3 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(hi), true);
  typename ActTraits<T>::vec8 r;
  r[0] = round_to<T>(p0.x * s); r[1] = round_to<T>(p0.y * s);
  r[2] = round_to<T>(p1.x * s); r[3] = round_to<T>(p1.y * s);
  r[4] = round_to<T>(p2.x * s); r[5] = round_to<T>(p2.y * s);
  r[6] = round_to<T>(p3.x * s); r[7] = round_to<T>(p3.y * s);
  return r;
}

// ------------------------------------------------------------------ division
//
// n / d for 32-bit n by a divisor d >= 1 fixed at launch (Granlund &
// Montgomery, "Division by invariant integers using multiplication", 1994):
// q = (umulhi(n, m) + n) >> l with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1.
struct FastDiv {
  uint32_t m, l, d;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
  return FastDiv{static_cast<uint32_t>(m), l, d};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, FastDiv f) {
  const uint64_t t = static_cast<uint64_t>(__umulhi(n, f.m)) + n;
  return static_cast<uint32_t>(t >> f.l);
}

// ------------------------------------------------------------------ buffer loads
//
// Raw buffer loads through a wave-uniform resource descriptor: an access at or
// beyond `bytes` from the base returns zero instead of faulting, so tails and
// masked lanes need no branch around the load (branches there make the
// compiler wait for every outstanding load).  Offsets are 32-bit.

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // any offset >= every `bytes` used here

// `base` and `bytes` must be the same on every lane of the wave.  They are
// passed through readfirstlane so the compiler knows it too: a descriptor it
// cannot prove uniform is wrapped in a per-lane loop around every load.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* up = reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
  // third descriptor dword for raw (untyped, unswizzled) buffers on gfx9-family GPUs
  return __builtin_amdgcn_make_buffer_rsrc(up, static_cast<short>(0), static_cast<int>(n), 0x00020000);
}
// The offsets passed below are often `cond ? offset : kOutOfRange`; left as
// is, the compiler may turn that select into two branches, each with its own
// load, and then wait for all loads where they join.  Pinning the offset in a
// VGPR first keeps it a select (the barrier emits no instruction).
__device__ __forceinline__ uint32_t vgpr(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ u32x4 buf_load_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, vgpr(off), 0, 0));
}
// Per-lane offset `voff` plus a wave-uniform offset `soff` (a scalar
// register: no per-lane address arithmetic).  The caller keeps voff + soff +
// 16 inside the bytes the lane may read: only `voff` is guaranteed to take
// part in the range check.
__device__ __forceinline__ u32x4 buf_load_b128_so(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 buf_load_b64(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, vgpr(off), 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_b32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, vgpr(off), 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u16(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, vgpr(off), 0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
// LDS pointers for reads whose addresses are computed in 32 bits
typedef __attribute__((address_space(3))) const unsigned char* lds_cbytes;
typedef __attribute__((address_space(3))) const u32x4 lds_u32x4;

// Direct buffer -> LDS load of SIZE bytes per lane: lane l writes lds +
// SIZE l (lds must be wave-uniform); offsets past the descriptor's range
// write zeros.  The compiler does not track the LDS write: the caller waits
// for it (vmcnt) before reading the data.
template <int SIZE>
__device__ __forceinline__ void buf_load_lds(rsrc_t r, uint32_t voff, void* lds) {
  static_assert(SIZE == 16 || SIZE == 4, "direct load size");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds), 16, vgpr(voff), 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds), 4, vgpr(voff), 0, 0, 0);
}

// 16-byte global load of 8 T values, reinterpreted as the MFMA operand type.
template <typename V>
__device__ __forceinline__ V load16(const void* p) {
  return *reinterpret_cast<const V*>(p);
}

}  // namespace fp4w

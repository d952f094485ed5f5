// Decode GEMV (1 <= M <= 8) for weight-only FP4 and FP8, on MFMA.
//
// Memory-bound: every packed weight byte and scale byte is read from HBM once
// with 16-byte loads; activations (M x K, at most 80 KiB) are re-read from L2
// only once per 16 output columns.
//
// Structure (per wave64; see [FP4 doc] §4 "Tensor-core sub-path" and [FP8
// doc] §4.1 for the pages' CUDA mma.m16n8k16 version, which this re-derives
// for the CDNA4 v_mfma_f32_16x16x32_{bf16,f16} operand layout):
//  * one MFMA tile = 16 output columns n (the B operand: lane l supplies
//    column l % 16) x 16 activation rows m (the A operand, rows >= M are
//    zero) x 32 k-slots, lane group g = l / 16 supplying k-slots 8g..8g+7;
//  * K is a reduction axis, so it is permuted: in window w (128 k), lane group
//    g owns the contiguous chunk c = 4w + g of 32 k.  One 16-byte load gives
//    that lane its 32 FP4 codes (one uint4 per lane per window, as on the
//    page), and MFMA i (i = 0..3) takes k = 32c + 8i .. 32c + 8i + 7 for both
//    operands;
//  * FP4: the E4M3 block scale is folded into the decoded weight before the
//    MFMA, exactly (E2M1 x E4M3 needs <= 6 significand bits: [FP4 doc] §4);
//    weight_scale_2 is applied once in the epilogue, bias fused there too
//    ([FP4 doc] §4);
//  * FP8: E4M3 -> T is exact, but the FP32 block scale is not, so each
//    window (which lies inside one scale block, block_size % 128 == 0) is
//    accumulated in a fresh MFMA accumulator and then scaled in FP32;
//  * KS waves of a workgroup split the K windows (the page's KSplit) and are
//    reduced through LDS; R column tiles per wave share one activation load.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"

#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

template <typename V>
__device__ __forceinline__ V zero_vec() {
  V v;
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0;
  return v;
}

// Activations of one lane for one chunk: A[m][32c .. 32c + 31] (4 x 16 bytes).
template <typename T, typename V>
__device__ __forceinline__ void load_act(const T* __restrict__ arow, int c, bool ok, V (&a)[4]) {
  if (ok) {
    const T* p = arow + 32 * c;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = load16<V>(p + 8 * i);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = zero_vec<V>();
  }
}

// --------------------------------------------------------------------- FP4

template <typename T, int R, int KS>
__global__ __launch_bounds__(64 * KS) void fp4_gemv_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const uint8_t* __restrict__ ws,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int M, int N,
    int K) {
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int n_base = blockIdx.x * (16 * R);
  const int NC = K >> 5;          // 32-k chunks
  const int NW = (NC + 3) >> 2;   // 128-k windows
  const int half_k = K >> 1;      // bytes per packed row
  const int cols = K >> 4;        // scale bytes per row

  const bool m_ok = li < M;
  const T* arow = A + static_cast<size_t>(m_ok ? li : 0) * K;
  const uint8_t* brow[R];
  const uint8_t* srow[R];
  bool n_ok[R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int n = n_base + 16 * t + li;
    n_ok[t] = n < N;
    const size_t nn = n_ok[t] ? n : 0;
    brow[t] = B + nn * half_k;
    srow[t] = ws + nn * cols;
  }

  f32x4 acc[R];
#pragma unroll
  for (int t = 0; t < R; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  // software pipeline: raw data of the next window is in flight while the
  // current one is decoded and multiplied
  V a_cur[4];
  u32x4 w_cur[R];
  uint32_t s_cur[R];
  int w = wave;
  auto fetch = [&](int win, V (&a)[4], u32x4 (&wq)[R], uint32_t (&sc)[R]) {
    const int c = 4 * win + g;
    const bool c_ok = (win < NW) && (c < NC);
    load_act<T, V>(arow, c, m_ok && c_ok, a);
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if (n_ok[t] && c_ok) {
        wq[t] = *reinterpret_cast<const u32x4*>(brow[t] + 16 * c);
        sc[t] = *reinterpret_cast<const uint16_t*>(srow[t] + 2 * c);
      } else {
        wq[t] = u32x4{0u, 0u, 0u, 0u};
        sc[t] = 0u;
      }
    }
  };
  fetch(w, a_cur, w_cur, s_cur);
  for (; w < NW; w += KS) {
    V a_nxt[4];
    u32x4 w_nxt[R];
    uint32_t s_nxt[R];
    fetch(w + KS, a_nxt, w_nxt, s_nxt);
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const typename Tr::scale_t s0 = Tr::make_scale(e4m3_to_f32<0>(s_cur[t]));
      const typename Tr::scale_t s1 = Tr::make_scale(e4m3_to_f32<1>(s_cur[t]));
      const V b0 = Tr::decode8(w_cur[t].x, s0);
      const V b1 = Tr::decode8(w_cur[t].y, s0);
      const V b2 = Tr::decode8(w_cur[t].z, s1);
      const V b3 = Tr::decode8(w_cur[t].w, s1);
      acc[t] = Tr::mfma(a_cur[0], b0, acc[t]);
      acc[t] = Tr::mfma(a_cur[1], b1, acc[t]);
      acc[t] = Tr::mfma(a_cur[2], b2, acc[t]);
      acc[t] = Tr::mfma(a_cur[3], b3, acc[t]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a_cur[i] = a_nxt[i];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      w_cur[t] = w_nxt[t];
      s_cur[t] = s_nxt[t];
    }
  }

  // K-split reduction through LDS, then the epilogue on wave 0.
  // Accumulator layout: lane (li, g) holds column n = n_base + 16t + li and
  // rows m = 4g + r, r = 0..3.
  if (KS > 1) {
    __shared__ f32x4 red[KS][R][64];
#pragma unroll
    for (int t = 0; t < R; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      f32x4 s = red[0][t][lane];
#pragma unroll
      for (int v = 1; v < KS; ++v) s += red[v][t][lane];
      acc[t] = s;
    }
  }
  const float ws2 = *ws2p;
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int n = n_base + 16 * t + li;
    if (!n_ok[t]) continue;
    const float b = bias ? static_cast<float>(bias[n]) : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      if (m < M) Y[static_cast<size_t>(m) * N + n] = round_to<T>(fmaf(acc[t][r], ws2, b));
    }
  }
}

// --------------------------------------------------------------------- FP8

template <typename T, int R, int KS>
__global__ __launch_bounds__(64 * KS) void fp8_gemv_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const float* __restrict__ bscale,
    const T* __restrict__ bias, T* __restrict__ Y, int M, int N, int K, int bs, int cols) {
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int n_base = blockIdx.x * (16 * R);
  const int NW = K >> 7;  // 128-k windows (K % 128 == 0)

  const bool m_ok = li < M;
  const T* arow = A + static_cast<size_t>(m_ok ? li : 0) * K;
  const uint8_t* brow[R];
  const float* srow[R];
  bool n_ok[R];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int n = n_base + 16 * t + li;
    n_ok[t] = n < N;
    const size_t nn = n_ok[t] ? n : 0;
    brow[t] = B + nn * K;
    srow[t] = bscale + nn * cols;
  }
  f32x4 acc[R];
#pragma unroll
  for (int t = 0; t < R; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  V a_cur[4];
  u32x4 w_cur[R][2];
  float s_cur[R];
  auto fetch = [&](int win, V (&a)[4], u32x4 (&wq)[R][2], float (&sc)[R]) {
    const int c = 4 * win + g;
    const bool ok = win < NW;
    load_act<T, V>(arow, c, m_ok && ok, a);
    // every k of window `win` lies in scale column min(128 win / bs, cols - 1)
    const int col = ok ? min((128 * win) / bs, cols - 1) : 0;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      if (n_ok[t] && ok) {
        const u32x4* p = reinterpret_cast<const u32x4*>(brow[t] + 32 * c);
        wq[t][0] = p[0];
        wq[t][1] = p[1];
        sc[t] = srow[t][col];
      } else {
        wq[t][0] = u32x4{0u, 0u, 0u, 0u};
        wq[t][1] = u32x4{0u, 0u, 0u, 0u};
        sc[t] = 0.0f;
      }
    }
  };
  int w = wave;
  fetch(w, a_cur, w_cur, s_cur);
  for (; w < NW; w += KS) {
    V a_nxt[4];
    u32x4 w_nxt[R][2];
    float s_nxt[R];
    fetch(w + KS, a_nxt, w_nxt, s_nxt);
#pragma unroll
    for (int t = 0; t < R; ++t) {
      const V b0 = Tr::decode8_fp8(w_cur[t][0].x, w_cur[t][0].y);
      const V b1 = Tr::decode8_fp8(w_cur[t][0].z, w_cur[t][0].w);
      const V b2 = Tr::decode8_fp8(w_cur[t][1].x, w_cur[t][1].y);
      const V b3 = Tr::decode8_fp8(w_cur[t][1].z, w_cur[t][1].w);
      f32x4 blk = f32x4{0.f, 0.f, 0.f, 0.f};
      blk = Tr::mfma(a_cur[0], b0, blk);
      blk = Tr::mfma(a_cur[1], b1, blk);
      blk = Tr::mfma(a_cur[2], b2, blk);
      blk = Tr::mfma(a_cur[3], b3, blk);
      // lane holds column n (one scale) and rows 4g..4g+3
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[t][r] = fmaf(blk[r], s_cur[t], acc[t][r]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a_cur[i] = a_nxt[i];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      w_cur[t][0] = w_nxt[t][0];
      w_cur[t][1] = w_nxt[t][1];
      s_cur[t] = s_nxt[t];
    }
  }
  if (KS > 1) {
    __shared__ f32x4 red[KS][R][64];
#pragma unroll
    for (int t = 0; t < R; ++t) red[wave][t][lane] = acc[t];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      f32x4 s = red[0][t][lane];
#pragma unroll
      for (int v = 1; v < KS; ++v) s += red[v][t][lane];
      acc[t] = s;
    }
  }
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int n = n_base + 16 * t + li;
    if (!n_ok[t]) continue;
    const float b = bias ? static_cast<float>(bias[n]) : 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 4 * g + r;
      if (m < M) Y[static_cast<size_t>(m) * N + n] = round_to<T>(acc[t][r] + b);
    }
  }
}

// --------------------------------------------------------------------- launch

// Launch shape: about 2048+ waves in flight (8 per CU on 256 CUs) so the HBM
// pipe stays full, KS limited by the number of windows.
struct GemvShape {
  int R, KS;
};

GemvShape pick_shape(int64_t N, int64_t windows) {
  const int64_t tiles = (N + 15) / 16;
  GemvShape s{1, 1};
  if (tiles >= 4096) s.R = 2;
  const int64_t groups = (tiles + s.R - 1) / s.R;
  while (s.KS < 8 && groups * s.KS < 2048 && windows >= 2 * s.KS * 2) s.KS *= 2;
  return s;
}

template <typename T, int R, int KS>
void launch_fp4_t(const MatmulArgs& a) {
  const int grid = static_cast<int>((a.N + 16 * R - 1) / (16 * R));
  hipLaunchKernelGGL((fp4_gemv_kernel<T, R, KS>), dim3(grid), dim3(64 * KS), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.A), a.B,
                     static_cast<const uint8_t*>(a.scales), a.ws2, static_cast<const T*>(a.bias),
                     static_cast<T*>(a.Y), static_cast<int>(a.M), static_cast<int>(a.N),
                     static_cast<int>(a.K));
}

template <typename T, int R, int KS>
void launch_fp8_t(const MatmulArgs& a) {
  const int grid = static_cast<int>((a.N + 16 * R - 1) / (16 * R));
  hipLaunchKernelGGL((fp8_gemv_kernel<T, R, KS>), dim3(grid), dim3(64 * KS), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.A), a.B,
                     static_cast<const float*>(a.scales), static_cast<const T*>(a.bias),
                     static_cast<T*>(a.Y), static_cast<int>(a.M), static_cast<int>(a.N),
                     static_cast<int>(a.K), static_cast<int>(a.block_size),
                     static_cast<int>(a.scale_cols));
}

template <typename T, bool FP8>
void launch_any(const MatmulArgs& a, GemvShape s) {
#define FP4W_GEMV_CASE(R_, KS_)                                        \
  if (s.R == R_ && s.KS == KS_) {                                      \
    if (FP8) launch_fp8_t<T, R_, KS_>(a); else launch_fp4_t<T, R_, KS_>(a); \
    return;                                                            \
  }
  FP4W_GEMV_CASE(1, 1) FP4W_GEMV_CASE(1, 2) FP4W_GEMV_CASE(1, 4) FP4W_GEMV_CASE(1, 8)
  FP4W_GEMV_CASE(2, 1) FP4W_GEMV_CASE(2, 2) FP4W_GEMV_CASE(2, 4) FP4W_GEMV_CASE(2, 8)
#undef FP4W_GEMV_CASE
}

}  // namespace

int launch_fp4_gemv(const MatmulArgs& a) {
  if (a.N > 0x7fffffff || a.K > 0x7fffffff || a.N * (a.K / 2) > (int64_t(1) << 40)) return -1;
  const GemvShape s = pick_shape(a.N, (a.K / 32 + 3) / 4);
  if (a.act == Act::BF16) launch_any<__bf16, false>(a, s);
  else launch_any<_Float16, false>(a, s);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fp8_gemv(const MatmulArgs& a) {
  if (a.N > 0x7fffffff || a.K > 0x7fffffff) return -1;
  const GemvShape s = pick_shape(a.N, a.K / 128);
  if (a.act == Act::BF16) launch_any<__bf16, true>(a, s);
  else launch_any<_Float16, true>(a, s);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace fp4w

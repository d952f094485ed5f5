// Fused prefill GEMM for weight-only FP4 and FP8 (M > 8), on MFMA.
//
// The pages' prefill path expands B into an [N, K] FP16/BF16 scratch tensor,
// runs cuBLAS on it and adds the bias in a third kernel ([FP4 doc] §5; [Blog],
// where that expansion took 46.9 % of H200 prefill GPU time and the blog's
// closing questions ask whether the scratch must exist at all).  Here the
// packed weights are decoded straight into MFMA operands in registers, so no
// scratch is written or re-read, and the tensor scale and bias are applied in
// the epilogue.
//
// Tiling (gfx950, wave64):
//  * workgroup tile (128 WM) (M) x 256 (N) x 64 (K per step), WM x 4 waves,
//    each wave 128 x 64 = 8 x 4 tiles of v_mfma_f32_16x16x32 (FP4: WM = 2,
//    two waves per SIMD; FP8: WM = 1, one wave per SIMD, whose 512 registers
//    hold both the running sum and the current scale block's sum);
//  * the activation tile (128 WM x 64 of T) is staged in LDS, double
//    buffered, 16-byte chunks XOR-swizzled by row so the ds_read_b128 of an
//    MFMA operand is bank-conflict free;
//  * weights go global -> registers directly: each wave owns 64 columns, so
//    its packed bytes are private to it; lane (column li, k-group g) loads the
//    16 consecutive k of its column in this step (8 bytes FP4 / 16 bytes FP8),
//    which is one whole 16-element FP4 scale block (K permuted per lane as in
//    the GEMV: the same permutation is applied to both operands);
//  * FP4: the E4M3 scale is folded into the decoded BF16/FP16 operand (exact,
//    [FP4 doc] §4); the FP32 weight_scale_2 multiplies the FP32 accumulator
//    once in the epilogue, together with the bias;
//  * FP8: E4M3 -> T is exact but the FP32 block scale is not, so the steps of
//    one scale block (block_size % 64 == 0) are accumulated in a separate
//    MFMA accumulator, which is then added to the running sum scaled in FP32.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [Blog]    = "ONNX Runtime #32128 - Why Dequantizing 4-Bit Weights Became the
//             Most Expensive Kernel in H200 Prefill"

#include <hip/hip_runtime.h>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr int BN = 256, BK = 64;
constexpr int kLdsRow = BK;  // elements per LDS row (no padding: XOR swizzle)

__device__ __forceinline__ int lds_index(int row, int chunk) {
  return row * kLdsRow + ((chunk ^ (row & 7)) << 3);
}

template <typename T, bool FP8, int WM>
__global__ __launch_bounds__(256 * WM) void gemm_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const void* __restrict__ scales,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int M, int N,
    int K, int cols, int bs, int tiles_m) {
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  constexpr int BM = 128 * WM;
  __shared__ __attribute__((aligned(16))) T As[2][BM * kLdsRow];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;
  const int tm = blockIdx.x % tiles_m, tn = blockIdx.x / tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  // activation staging: 4 chunks of 16 bytes per thread per step
  const T* a_src[4];
  int a_dst[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (tid >> 3) + 32 * WM * j;
    const int gm = min(m0 + row, M - 1);
    a_src[j] = A + static_cast<size_t>(gm) * K + (tid & 7) * 8;
    a_dst[j] = lds_index(row, tid & 7);
  }
  // this lane's 4 weight columns (one per 16-wide N sub-tile)
  const uint8_t* b_src[4];
  const void* s_src[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int n = min(n0 + 64 * wn + 16 * ns + li, N - 1);
    if (FP8) {
      b_src[ns] = B + static_cast<size_t>(n) * K + 16 * g;
      s_src[ns] = static_cast<const float*>(scales) + static_cast<size_t>(n) * cols;
    } else {
      b_src[ns] = B + static_cast<size_t>(n) * (K / 2) + 8 * g;
      s_src[ns] = static_cast<const uint8_t*>(scales) + static_cast<size_t>(n) * cols + g;
    }
  }

  f32x4 acc[8][4];
  f32x4 blk[FP8 ? 8 : 1][4];  // FP8: sum over the current scale block
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < (FP8 ? 8 : 1); ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) blk[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nsteps = K / BK;
  u32x4 a_reg[4];
  // raw weights of one step: FP4 2 dwords per column, FP8 4 dwords
  u32x4 b_cur[4], b_nxt[4];
  float s_cur[4], s_nxt[4];

  auto load_a = [&](int step) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a_reg[j] = *reinterpret_cast<const u32x4*>(a_src[j] + step * BK);
  };
  auto store_a = [&](int stage) {
#pragma unroll
    for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&As[stage][a_dst[j]]) = a_reg[j];
  };
  auto load_b = [&](int step, u32x4 (&bw)[4], float (&sc)[4]) {
    const int k0 = step * BK;
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      if (FP8) {
        bw[ns] = *reinterpret_cast<const u32x4*>(b_src[ns] + k0);
        const int col = min(k0 / bs, cols - 1);
        sc[ns] = static_cast<const float*>(s_src[ns])[col];
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(b_src[ns] + k0 / 2);
        bw[ns] = u32x4{v.x, v.y, 0u, 0u};
        sc[ns] = e4m3_to_f32<0>(static_cast<const uint8_t*>(s_src[ns])[k0 / 16]);
      }
    }
  };

  load_a(0);
  store_a(0);
  load_b(0, b_cur, s_cur);
  __syncthreads();

  for (int step = 0; step < nsteps; ++step) {
    const int cur = step & 1;
    const bool more = step + 1 < nsteps;
    if (more) {
      load_a(step + 1);
      load_b(step + 1, b_nxt, s_nxt);
    }
    const T* as = As[cur];
    if (!FP8) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        V bop[4];
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
          bop[ns] = Tr::decode8(s == 0 ? b_cur[ns].x : b_cur[ns].y, Tr::make_scale(s_cur[ns]));
#pragma unroll
        for (int ms = 0; ms < 8; ++ms) {
          const int row = 128 * wm + 16 * ms + li;
          const V aop = *reinterpret_cast<const V*>(&as[lds_index(row, 2 * g + s)]);
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = Tr::mfma(aop, bop[ns], acc[ms][ns]);
        }
      }
    } else {
      V bop[2][4];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        bop[0][ns] = Tr::decode8_fp8(b_cur[ns].x, b_cur[ns].y);
        bop[1][ns] = Tr::decode8_fp8(b_cur[ns].z, b_cur[ns].w);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
#pragma unroll
        for (int ms = 0; ms < 8; ++ms) {
          const int row = 128 * wm + 16 * ms + li;
          const V aop = *reinterpret_cast<const V*>(&as[lds_index(row, 2 * g + s)]);
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) blk[ms][ns] = Tr::mfma(aop, bop[s][ns], blk[ms][ns]);
        }
      }
      // close the scale block after its last step: running sum += block sum * scale
      const int k0 = step * BK;
      const bool flush = !more || min((k0 + BK) / bs, cols - 1) != min(k0 / bs, cols - 1);
      if (flush) {
#pragma unroll
        for (int ms = 0; ms < 8; ++ms)
#pragma unroll
          for (int ns = 0; ns < 4; ++ns) {
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[ms][ns][r] = fmaf(blk[ms][ns][r], s_cur[ns], acc[ms][ns][r]);
            blk[ms][ns] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
    if (more) {
      store_a(cur ^ 1);
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        b_cur[ns] = b_nxt[ns];
        s_cur[ns] = s_nxt[ns];
      }
    }
    __syncthreads();
  }

  // epilogue: lane (li, g) holds columns n0 + 64 wn + 16 ns + li and rows
  // m0 + 128 wm + 16 ms + 4 g + r
  const float ws2 = FP8 ? 1.0f : *ws2p;
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int n = n0 + 64 * wn + 16 * ns + li;
    if (n >= N) continue;
    const float b = bias ? static_cast<float>(bias[n]) : 0.0f;
#pragma unroll
    for (int ms = 0; ms < 8; ++ms) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + 128 * wm + 16 * ms + 4 * g + r;
        if (m < M) {
          const float y = FP8 ? acc[ms][ns][r] + b : fmaf(acc[ms][ns][r], ws2, b);
          Y[static_cast<size_t>(m) * N + n] = round_to<T>(y);
        }
      }
    }
  }
}

template <typename T, bool FP8>
int launch(const MatmulArgs& a) {
  constexpr int WM = FP8 ? 1 : 2;
  constexpr int BM = 128 * WM;
  if (a.M > 0x7fffffff || a.N > 0x7fffffff || a.K > 0x7fffffff) return -1;
  const int64_t tiles_m = (a.M + BM - 1) / BM, tiles_n = (a.N + BN - 1) / BN;
  if (tiles_m * tiles_n > 0x7fffffff) return -1;
  hipLaunchKernelGGL((gemm_kernel<T, FP8, WM>), dim3(static_cast<unsigned>(tiles_m * tiles_n)),
                     dim3(256 * WM), 0, static_cast<hipStream_t>(a.stream),
                     static_cast<const T*>(a.A), a.B, a.scales, a.ws2,
                     static_cast<const T*>(a.bias), static_cast<T*>(a.Y), static_cast<int>(a.M),
                     static_cast<int>(a.N), static_cast<int>(a.K), static_cast<int>(a.scale_cols),
                     static_cast<int>(a.block_size), static_cast<int>(tiles_m));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_fp4_gemm(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch<__bf16, false>(a) : launch<_Float16, false>(a);
}

int launch_fp8_gemm(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch<__bf16, true>(a) : launch<_Float16, true>(a);
}

}  // namespace fp4w

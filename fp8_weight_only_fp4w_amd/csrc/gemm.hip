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

#include <type_traits>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr int BN = 256, BK = 64;
constexpr int kLdsRow = BK;  // elements per LDS row (no padding: XOR swizzle)

// 16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 7): the 16 rows read
// by a 16-lane group at one logical chunk land in 16 distinct 16-byte slots of
// a 256-byte LDS line (rows are 128 bytes), so ds_read_b128 is conflict free.
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_index(int row, int chunk) {
  return row * kLdsRow + ((chunk ^ lds_swz(row)) << 3);
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

// FP4 prefill GEMM, large tiles.  Workgroup 256 (M) x 256 (N) x 64 (K per
// step), 8 waves in a 2 (M) x 4 (N) grid, each wave 128 x 64 = 8 x 4 tiles of
// v_mfma_f32_16x16x32 (128 FP32 accumulators per lane), two waves per SIMD:
// a wave's weight decode (vector ALU) runs while the other wave's MFMAs
// occupy the matrix core (one wave alone does not overlap the two).
//  * Every operand tile (activations, packed weights, scale bytes) moves
//    global -> LDS by direct loads (global_load_lds: no registers), three
//    stages deep: the tiles of step t + 2 are requested during step t, so a
//    load has two steps of MFMA work to arrive.  The only wait is, at the end
//    of each step, for the tiles of the next step (loads complete in order).
//  * LDS layout per stage: activations [256 rows][64] of T with 16-byte chunks
//    XOR-swizzled by row (the swizzle is applied to the global addresses,
//    since one direct load writes 1 KiB contiguously), packed weights
//    [256 columns][32 bytes], scale bytes [256 columns][4].
//  * Lane (li, g) takes k 16g .. 16g + 15 of each step for both operands
//    (one 16-element scale block), split in two 8-k halves over two MFMAs;
//    the E4M3 scale is folded into the decoded BF16/FP16 operand (exact).
//  * Tile order: workgroups are dispatched round-robin over the 8 XCDs, each
//    with its own L2, so the workgroup index is remapped to give every XCD a
//    contiguous range of tiles, walked in groups of 8 tile rows.
constexpr int L_BM = 256, L_BN = 256;

template <typename T, bool FP8>
struct LargeStage {
  T a[L_BM * kLdsRow];               // 32 KiB
  uint8_t b[L_BN * (FP8 ? 64 : 32)];  // 16 / 8 KiB of weight bytes
  uint8_t s[L_BN * 4];               // 1 KiB: 4 E4M3 bytes or one FP32 scale per column
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// direct 16-byte (or 4-byte) global -> LDS load: lane l writes lds + l * size
template <int SIZE>
__device__ __forceinline__ void load_lds(const void* gptr, void* lds) {
  static_assert(SIZE == 16 || SIZE == 4, "direct load size");
  if constexpr (SIZE == 16)
    __builtin_amdgcn_global_load_lds(gptr, (lds_ptr_t)(lds), 16, 0, 0);
  else
    __builtin_amdgcn_global_load_lds(gptr, (lds_ptr_t)(lds), 4, 0, 0);
}

// wait until at most N vector-memory loads are in flight and every LDS access
// has completed, then barrier (the compiler fences keep LDS accesses on
// their side of it)
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));  // lgkmcnt(0), vmcnt(N)
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

template <typename T, bool FP8>
__global__ __launch_bounds__(512) void gemm_large_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const uint8_t* __restrict__ scales,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int M, int N,
    int K, int cols, int bs, int tiles_m, int tiles_n) {
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  typedef LargeStage<T, FP8> Stage;
  __shared__ __attribute__((aligned(16))) Stage st[3];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  const int wm = wave >> 2, wn = wave & 3;

  // tile index: contiguous range per XCD, then groups of 8 tile rows
  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int first_m = (t / per_group) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int m0 = tm * L_BM, n0 = tn * L_BN;

  // Direct-load sources of this lane (element / byte offsets, step 0).
  // Activations: instruction j of wave w writes rows 8q .. 8q + 7 of the
  // stage, q = 8j + w; lane l lands in row 8q + l / 8, LDS chunk l % 8, which
  // holds global chunk (l % 8) ^ (l / 8) under the swizzle.
  int a_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = 8 * (8 * j + wave) + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_swz(row);
    a_off[j] = min(m0 + row, M - 1) * K + 8 * chunk;
  }
  // Weights.  FP4 (32 bytes per column and step): instruction j of wave w
  // covers columns 32q .. 32q + 31, q = w; lane l lands in column 32q + l / 2,
  // 16-byte piece l % 2.  FP8 (64 bytes): q = 8j + w, 16 columns per
  // instruction, lane l in column 16q + l / 4, piece l % 4.  Pieces are
  // swizzled with the column (global piece = LDS piece ^ bit pattern of the
  // column) so the 16 columns read by a 16-lane group fall in distinct banks.
  constexpr int kBBytes = FP8 ? 64 : 32;            // per column and step
  constexpr int kBLoads = FP8 ? 2 : 1;              // direct loads per wave and step
  constexpr int kColsPerLoad = 1024 / kBBytes;      // columns per direct load
  constexpr int kPieces = kBBytes / 16;
  auto b_swz = [](int col) { return FP8 ? (col & 3) : ((col >> 3) & 1); };
  const size_t b_row = FP8 ? static_cast<size_t>(K) : static_cast<size_t>(K / 2);
  int b_off[kBLoads];
#pragma unroll
  for (int j = 0; j < kBLoads; ++j) {
    const int col = kColsPerLoad * (8 * j + wave) + lane / kPieces;
    const int piece = (lane % kPieces) ^ b_swz(col);
    b_off[j] = min(n0 + col, N - 1) * static_cast<int>(b_row) + 16 * piece;
  }
  // scales: wave w covers columns 64 (w % 4) .. + 63, 4 bytes each: the 4
  // E4M3 bytes of the step (FP4) or the FP32 scale of the step's block (FP8;
  // block_size % 64 == 0, so a step lies in one block).  Waves 4..7 repeat
  // waves 0..3: identical data to identical addresses, which keeps the number
  // of loads per wave uniform.
  const int s_col = 64 * (wave & 3) + lane;
  const int s_off = min(n0 + s_col, N - 1) * cols;  // elements (bytes FP4, floats FP8)

  const int nsteps = K / BK;
  auto issue = [&](int step, Stage& st) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      load_lds<16>(A + a_off[j] + step * BK, &st.a[(8 * j + wave) * 8 * kLdsRow]);
#pragma unroll
    for (int j = 0; j < kBLoads; ++j)
      load_lds<16>(B + b_off[j] + static_cast<size_t>(step) * (FP8 ? BK : BK / 2), &st.b[(8 * j + wave) * 1024]);
    if constexpr (FP8) {
      const int col = min(step * BK / bs, cols - 1);
      load_lds<4>(reinterpret_cast<const float*>(scales) + s_off + col, &st.s[64 * (wave & 3) * 4]);
    } else {
      load_lds<4>(scales + s_off + step * (BK / 16), &st.s[64 * (wave & 3) * 4]);
    }
  };
  constexpr int kLoadsPerStep = 4 + kBLoads + 1;  // direct loads per wave and step

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage& st) {
    // lane (li, g): k 16g .. 16g + 15 of its 4 columns (FP4 8 bytes, FP8 16)
    u32x4 bw[4];
    float sc[4];
#pragma unroll
    for (int ns = 0; ns < 4; ++ns) {
      const int col = 64 * wn + 16 * ns + li;
      if constexpr (FP8) {
        bw[ns] = *reinterpret_cast<const u32x4*>(&st.b[col * 64 + 16 * (g ^ b_swz(col))]);
        sc[ns] = *reinterpret_cast<const float*>(&st.s[col * 4]);
      } else {
        const u32x2 v = *reinterpret_cast<const u32x2*>(&st.b[col * 32 + 16 * ((g >> 1) ^ b_swz(col)) + 8 * (g & 1)]);
        bw[ns].x = v.x;
        bw[ns].y = v.y;
        sc[ns] = e4m3_to_f32<0>(st.s[col * 4 + g]);
      }
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      V aop[8];
#pragma unroll
      for (int ms = 0; ms < 8; ++ms)
        aop[ms] = *reinterpret_cast<const V*>(&st.a[lds_index(128 * wm + 16 * ms + li, 2 * g + s)]);
      V bop[4];
#pragma unroll
      for (int ns = 0; ns < 4; ++ns) {
        if constexpr (FP8)
          bop[ns] = decode8_fp8_scaled<T>(bw[ns][2 * s], bw[ns][2 * s + 1], sc[ns]);
        else
          bop[ns] = Tr::decode8(bw[ns][s], Tr::make_scale(sc[ns]));
      }
#pragma unroll
      for (int ms = 0; ms < 8; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns) acc[ms][ns] = Tr::mfma(aop[ms], bop[ns], acc[ms][ns]);
    }
  };

  auto do_step = [&](int step, const Stage& cur, Stage& ahead2) {
    const bool issue2 = step + 2 < nsteps;
    if (issue2) issue(step + 2, ahead2);
    compute(cur);
    if (issue2)
      wait_barrier<kLoadsPerStep>();  // the tiles of step + 1 have landed
    else
      wait_barrier<0>();
  };

  issue(0, st[0]);
  if (nsteps > 1) issue(1, st[1]);
  if (nsteps > 1)
    wait_barrier<kLoadsPerStep>();
  else
    wait_barrier<0>();
  for (int step = 0; step < nsteps; step += 3) {
    do_step(step, st[0], st[2]);
    if (step + 1 < nsteps) do_step(step + 1, st[1], st[0]);
    if (step + 2 < nsteps) do_step(step + 2, st[2], st[1]);
  }

  // Epilogue: lane (li, g) holds columns 64 wn + 16 ns + li and rows
  // 128 wm + 16 ms + 4 g + r of the tile.  Y = acc * ws2 + bias, rounded once
  // to T, is staged in LDS (the operand stages are free now) one 128-row half
  // at a time and written back in whole 16-byte row pieces; tiles on the
  // ragged edge, or outputs that are not 16-byte aligned, store element-wise.
  const float ws2 = FP8 ? 1.0f : *ws2p;
  constexpr int kOutPitch = L_BN + 8;  // elements per staged row (breaks bank aliasing)
  T* out = reinterpret_cast<T*>(&st[0]);
  const bool wide = (N % 8 == 0) && (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && n0 + L_BN <= N;
  float bsum[4];
#pragma unroll
  for (int ns = 0; ns < 4; ++ns) {
    const int n = min(n0 + 64 * wn + 16 * ns + li, N - 1);
    bsum[ns] = bias ? static_cast<float>(bias[n]) : 0.0f;
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if (wm == half) {
#pragma unroll
      for (int ms = 0; ms < 8; ++ms)
#pragma unroll
        for (int ns = 0; ns < 4; ++ns)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            out[(16 * ms + 4 * g + r) * kOutPitch + 64 * wn + 16 * ns + li] =
                round_to<T>(fmaf(acc[ms][ns][r], ws2, bsum[ns]));
    }
    __syncthreads();
    const int mrow0 = m0 + 128 * half;
    if (wide) {
      // 128 rows x 32 pieces of 16 bytes, 8 per thread
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int q = tid + 512 * i;
        const int row = q >> 5, piece = q & 31;
        if (mrow0 + row < M)
          *reinterpret_cast<u32x4*>(&Y[static_cast<size_t>(mrow0 + row) * N + n0 + 8 * piece]) =
              *reinterpret_cast<const u32x4*>(&out[row * kOutPitch + 8 * piece]);
      }
    } else {
      for (int q = tid; q < 128 * L_BN; q += 512) {
        const int row = q / L_BN, col = q % L_BN;
        if (mrow0 + row < M && n0 + col < N)
          Y[static_cast<size_t>(mrow0 + row) * N + n0 + col] = out[row * kOutPitch + col];
      }
    }
    __syncthreads();
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

template <typename T, bool FP8>
int launch_large(const MatmulArgs& a) {
  if (a.M > 0x7fffffff || a.N > 0x7fffffff || a.K > 0x7fffffff) return -1;
  // 32-bit element offsets inside the kernel
  const int64_t b_bytes = a.N * (FP8 ? a.K : a.K / 2);
  if (b_bytes >= (int64_t(1) << 31) || a.N * a.scale_cols >= (int64_t(1) << 31) ||
      static_cast<int64_t>(L_BM) * a.K >= (int64_t(1) << 31) || a.M * a.K >= (int64_t(1) << 31))
    return launch<T, FP8>(a);
  const int64_t tiles_m = (a.M + L_BM - 1) / L_BM, tiles_n = (a.N + L_BN - 1) / L_BN;
  if (tiles_m * tiles_n > 0x7fffffff) return -1;
  hipLaunchKernelGGL((gemm_large_kernel<T, FP8>), dim3(static_cast<unsigned>(tiles_m * tiles_n)), dim3(512), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.A), a.B,
                     static_cast<const uint8_t*>(a.scales), a.ws2, static_cast<const T*>(a.bias),
                     static_cast<T*>(a.Y), static_cast<int>(a.M), static_cast<int>(a.N), static_cast<int>(a.K),
                     static_cast<int>(a.scale_cols), static_cast<int>(a.block_size), static_cast<int>(tiles_m),
                     static_cast<int>(tiles_n));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fp4_gemm(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_large<__bf16, false>(a) : launch_large<_Float16, false>(a);
}

int launch_fp8_gemm(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_large<__bf16, true>(a) : launch_large<_Float16, true>(a);
}

}  // namespace fp4w

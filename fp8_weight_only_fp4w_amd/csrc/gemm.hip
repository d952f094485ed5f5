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
// One kernel, gemm_large_kernel, in three shapes (gfx950, wave64, 8 waves per
// workgroup, 64 K per step, v_mfma_f32_32x32x16 with FP32 accumulators):
//  * FP4 whole tiles: 128 (M) x 512 (N), the 8 waves side by side in N, each
//    128 x 64 = 4 x 2 MFMA tiles.  The E4M3 block scale is folded into the
//    decoded BF16/FP16 operand, which is exact (E2M1 x E4M3 needs 6
//    significand bits; [FP4 doc] §4); weight_scale_2 and the bias are applied
//    once in the epilogue.
//  * FP4 split tiles (the last, partial round of tiles): one workgroup takes
//    256 columns of a 128 x 512 tile, and its two wave groups take the two
//    halves of K (see SPLIT below).
//  * FP8: 128 x 256, waves in a 2 (M) x 4 (N) grid, each 64 x 64 = 2 x 2 MFMA
//    tiles.  E4M3 -> T is exact; the FP32 block scale is not representable in
//    the operand, so every scale block (block_size % 64 == 0) accumulates in
//    a fresh set of FP32 accumulators, which is then added to the running sum
//    multiplied by its b_scale in FP32 ([FP8 doc] §2: B_dq = e4m3 * b_scale).
//    The two sets take 128 registers per lane, which is why an FP8 wave holds
//    half the outputs of an FP4 wave.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"
// [Blog]    = "ONNX Runtime #32128 - Why Dequantizing 4-Bit Weights Became the
//             Most Expensive Kernel in H200 Prefill"

#include <hip/hip_runtime.h>

#include <type_traits>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr int BK = 64;
constexpr int kLdsRow = BK;  // elements per LDS row (no padding: XOR swizzle)

// 16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 7): the 16 rows read
// by a 16-lane group at one logical chunk land in 16 distinct 16-byte slots of
// a 256-byte LDS line (rows are 128 bytes), so ds_read_b128 is conflict free.
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_index(int row, int chunk) {
  return row * kLdsRow + ((chunk ^ lds_swz(row)) << 3);
}

// Common structure of the three shapes.  Waves w and w + 4 share a SIMD: a
// wave's weight decode (vector ALU) runs while the other wave's MFMAs occupy
// the matrix core.
//  * Every operand tile moves global -> LDS by direct loads (no registers).
//    What limits these loads is the number of L2 requests rather than their
//    bytes: a request carries one piece of at most 64 bytes of a line, so a
//    4- or 32-byte piece costs as much as a full one (measured: the 4-byte
//    scale pieces and 32-byte weight pieces of the first version of this
//    kernel took more load time than the activation tiles, which are 80 % of
//    the bytes).  So each operand is loaded in the largest contiguous pieces
//    its layout allows:
//     - activations: ring of 3 one-step stages [rows][64] of T (rows of 128
//       contiguous bytes);
//     - FP4 weights: ring of 2 slots of two steps each, 64 contiguous bytes
//       per column; FP8 weights: ring of 3 one-step stages, 64 bytes per
//       column;
//     - scales: ring of 2 slots of eight steps each, 32 contiguous bytes per
//       column (32 E4M3 bytes, or 8 FP32 block scales starting at the first
//       block of the slot).
//    Every load goes through a buffer descriptor (32-bit offsets, cheaper to
//    issue than 64-bit addresses) whose base is the workgroup's first row of
//    A and first column of B and of the scales, so any matrix size works;
//    pieces past the matrix read zeros.
//    The tiles of step t + 2 are requested during step t (FP4: spread over
//    its MFMA groups); the only wait is, at the end of each step, for the
//    tiles of step t + 1 (loads complete in order), then one barrier.  A slot
//    is refilled only after the barrier that ends its last reader's step.
//  * LDS layouts are XOR-swizzled in 16-byte pieces (applied on the global
//    side, since one direct load writes its 64 lanes' data contiguously), so
//    the operand reads of a 16-lane group hit distinct banks.
//  * Lane (c, h) takes column c of each 32-wide N tile and k 32h .. 32h + 31
//    of each step for both operands (FP4: two 16-element scale blocks, one
//    16-byte LDS read); MFMA i of the step takes k 32h + 8i .. 32h + 8i + 7.
//  * Tile order: workgroups are dispatched round-robin over the 8 XCDs, each
//    with its own L2, so the workgroup index is remapped to give every XCD a
//    contiguous range of tiles, walked in groups of tile rows.
//  * SPLIT (FP4): the tiles of a last round that would fill at most half the
//    CUs are launched separately, two workgroups per tile, 256 columns each;
//    waves 0-3 take the first half of K and waves 4-7 the second (stage rows
//    128 + r hold row r at k + K / 2; a weight slot holds one step of both
//    halves, a scale slot 4 steps of both), and the halves are added through
//    LDS before the epilogue.  That round then takes about half as long.
constexpr int kScaleSteps = 8;  // steps per scale slot

template <bool FP8, bool SPLIT>
struct LargeShape {
  static constexpr bool kWide = !FP8 && !SPLIT;
  static constexpr int kTM = 128;                   // output rows of a tile
  static constexpr int kTN = FP8 ? 256 : 512;       // output columns of a tile
  static constexpr int kSR = SPLIT ? 256 : 128;     // rows of an activation stage
  static constexpr int kSC = kWide ? 512 : 256;     // columns of a workgroup (weight and scale slots)
  static constexpr int kWaveM = FP8 ? 64 : 128;     // output rows of a wave
  static constexpr int kMS = kWaveM / 32;           // MFMA row tiles of a wave
  static constexpr int kAL = kSR / 64;              // activation loads per wave and step
  static constexpr int kBL = kSC / 128;             // weight loads per wave and slot
  static constexpr int kSL = kSC / 64;              // scale loads per wave and slot
  static constexpr int kGM = FP8 ? 4 : 8;           // tile rows per group of the tile order
};

template <typename T, bool FP8, bool SPLIT>
struct LargeLds {
  typedef LargeShape<FP8, SPLIT> Sh;
  T a[3][Sh::kSR * kLdsRow];                      // 3 x 16 KiB (split: 3 x 32 KiB)
  uint8_t b[FP8 || SPLIT ? 3 : 2][Sh::kSC * 64];  // FP8: 3 steps; FP4: 2 slots of 2 steps; split: 3 steps
  uint8_t s[2][Sh::kSC * 32];                     // 2 slots
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// v_mfma_f32_32x32x16 (BF16 / FP16 in, FP32 accumulate)
template <typename T>
__device__ __forceinline__ f32x16 mfma32(typename ActTraits<T>::vec8 a, typename ActTraits<T>::vec8 b, f32x16 c) {
  if constexpr (std::is_same<T, __bf16>::value)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
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

template <typename T, bool FP8, bool SPLIT>
__global__ __launch_bounds__(512) void gemm_large_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const uint8_t* __restrict__ scales,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int M, int N,
    int K, int cols, int bs, int tiles_m, int tiles_n, int t_first) {
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  __shared__ __attribute__((aligned(16))) LargeLds<T, FP8, SPLIT> L;
  typedef LargeShape<FP8, SPLIT> Sh;
  constexpr bool split = SPLIT;
  constexpr int SC = Sh::kSC;
  constexpr int MS = Sh::kMS;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // FP4 whole tiles: 8 waves in N.  Split: wave group wm takes half wm of K.
  // FP8: wave group wm takes rows 64 wm .. 64 wm + 63.
  const int wm = Sh::kWide ? 0 : wave >> 2, wn = Sh::kWide ? wave : wave & 3;

  // Whole tiles: workgroup b takes tile b (contiguous ranges per XCD, then
  // groups of GM tile rows).  Split launch (tiles t_first ..): two workgroups
  // take 256 columns each of one tile, and their two wave groups take the two
  // halves of K, which are added through LDS at the end.
  int t = blockIdx.x;
  if (SPLIT)
    t = t_first + t / 2;
  else if (gridDim.x % 8 == 0)
    t = (t % 8) * (gridDim.x / 8) + t / 8;
  constexpr int GM = Sh::kGM;
  const int per_group = GM * tiles_n;
  const int first_m = (t / per_group) * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int tm = first_m + (t % per_group) % gsize;
  const int tn = (t % per_group) / gsize;
  const int m0 = tm * Sh::kTM, n0 = tn * Sh::kTN + (SPLIT ? 256 * (blockIdx.x & 1) : 0);
  const int rows_m = min(Sh::kTM, M - m0);      // activation rows of this tile
  const int rows_n = max(min(SC, N - n0), 0);  // weight / scale rows of this workgroup

  // Activations: instruction j of wave w writes rows 8q .. 8q + 7 of the
  // stage, q = 8j + w; lane l lands in row 8q + l / 8, LDS chunk l % 8, which
  // holds global chunk (l % 8) ^ lds_swz(row).  Split: stage rows 128 + r hold
  // tile row r in the second half of K.  Rows past M repeat the last row
  // (their outputs are not stored).  Offsets are relative to row m0.
  int a_off[Sh::kAL];
#pragma unroll
  for (int j = 0; j < Sh::kAL; ++j) {
    const int row = 8 * (8 * j + wave) + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_swz(row);
    a_off[j] = split ? min(row & 127, rows_m - 1) * K + (row >> 7) * (K / 2) + 8 * chunk
                     : min(row, rows_m - 1) * K + 8 * chunk;
  }
  // Weights.  FP4 slot (two steps, 64 bytes per column, pieces 0-1 = the even
  // step, 2-3 = the odd step; split: one step, pieces 0-1 = its first half of
  // K, 2-3 = its second half): instruction j of wave w covers columns
  // 16q .. 16q + 15, q = 8j + w; lane l lands in column 16q + l / 4, LDS piece
  // l % 4, holding global piece (l % 4) ^ ((col >> 2) & 3).  FP8 stage (64
  // bytes per column): the same.
  const rsrc_t a_rsrc = make_rsrc(A + static_cast<size_t>(m0) * K,
                                  static_cast<uint32_t>(rows_m) * static_cast<uint32_t>(K) * 2u);
  const uint32_t b_row = FP8 ? static_cast<uint32_t>(K) : static_cast<uint32_t>(K / 2);
  auto b_swz = [](int col) { return (col >> 2) & 3; };
  uint32_t b_off[Sh::kBL];  // byte offset in the workgroup's descriptor
#pragma unroll
  for (int j = 0; j < Sh::kBL; ++j) {
    const int col = 16 * (8 * j + wave) + (lane >> 2);
    const int piece = (lane & 3) ^ b_swz(col);
    b_off[j] = static_cast<uint32_t>(col) * b_row + 16u * piece +
               (split && piece >= 2 ? static_cast<uint32_t>(K / 4 - 32) : 0u);
  }
  const rsrc_t b_rsrc = make_rsrc(B + static_cast<size_t>(n0) * b_row, static_cast<uint32_t>(rows_n) * b_row);
  // Scales: slot of 8 steps, 32 bytes per column (split: of 4 steps, 16 bytes
  // for each half of K).  Instruction j of wave w (4-byte pieces) covers
  // columns 8q .. 8q + 7, q = kSL w + j; lane l lands in column 8q + l / 8, LDS
  // piece (l % 8) / 4 (16-byte), holding global piece ((l % 8) / 4) ^
  // ((col >> 3) & 1).
  const uint32_t s_row = FP8 ? static_cast<uint32_t>(cols) * 4u : static_cast<uint32_t>(cols);
  uint32_t s_off[Sh::kSL];
#pragma unroll
  for (int j = 0; j < Sh::kSL; ++j) {
    const int col = 8 * (Sh::kSL * wave + j) + (lane >> 3);
    const int d = lane & 7;
    const int piece = (d >> 2) ^ ((col >> 3) & 1);
    s_off[j] = static_cast<uint32_t>(col) * s_row + 4u * (d & 3) +
               (split ? static_cast<uint32_t>(piece * (K / 32)) : 16u * piece);
  }
  const rsrc_t s_rsrc = make_rsrc(scales + static_cast<size_t>(n0) * s_row, static_cast<uint32_t>(rows_n) * s_row);
  const int spb = FP8 ? bs / BK : 1;  // steps per FP8 scale block (block_size % 64 == 0)
  // FP8: scale column of step u, and the first scale column of the slot
  // holding steps 8c .. 8c + 7
  auto step_col = [&](int u) { return min(u / spb, cols - 1); };
  auto slot_col = [&](int c) { return min(kScaleSteps * c / spb, cols - 1); };

  const int nsteps = split ? K / (2 * BK) : K / BK;
  const int sl = split ? kScaleSteps / 2 : kScaleSteps;  // steps per scale slot
  // loads a wave issues for step u: activations, weights (FP4: at even steps,
  // for the pair; split: every step), scales (at the first step of each slot)
  auto loads_for = [&](int u) {
    return Sh::kAL + (FP8 || split ? Sh::kBL : ((u & 1) ? 0 : Sh::kBL)) + (u % sl == 0 ? Sh::kSL : 0);
  };
  // part p (0 .. 3) of this wave's loads of step u
  auto issue_part = [&](int u, int p) {
    if (p < Sh::kAL)
      buf_load_lds<16>(a_rsrc, 2u * static_cast<uint32_t>(a_off[p] + u * BK), &L.a[u % 3][(8 * p + wave) * 8 * kLdsRow]);
    if (p < Sh::kBL) {
      if constexpr (FP8) {
        buf_load_lds<16>(b_rsrc, b_off[p] + static_cast<uint32_t>(u * BK), &L.b[u % 3][(8 * p + wave) * 1024]);
      } else {
        if (split)
          buf_load_lds<16>(b_rsrc, b_off[p] + 32u * u, &L.b[u % 3][(8 * p + wave) * 1024]);
        else if ((u & 1) == 0)
          buf_load_lds<16>(b_rsrc, b_off[p] + 32u * u, &L.b[(u >> 1) & 1][(8 * p + wave) * 1024]);
      }
    }
    if (u % sl == 0) {
      const int c = u / sl;
      const uint32_t base = FP8 ? 4u * static_cast<uint32_t>(slot_col(c)) : static_cast<uint32_t>(4 * sl * c);
      constexpr int kPer = Sh::kSL / 4;
#pragma unroll
      for (int j = kPer * p; j < kPer * (p + 1); ++j)
        buf_load_lds<4>(s_rsrc, s_off[j] + base, &L.s[c & 1][(Sh::kSL * wave + j) * 256]);
    }
  };
  auto issue = [&](int u) {
#pragma unroll
    for (int p = 0; p < 4; ++p) issue_part(u, p);
  };

  // lane (c32, h): column c32 of each 32-wide N tile, k half h of every step
  const int c32 = lane & 31, h = lane >> 5;
  const int a_row0 = Sh::kWaveM * wm;  // this wave's first row in an activation stage
  f32x16 acc[MS][2];
  // FP8: the current scale block's sum (fresh at the first step of a block)
  f32x16 blk[FP8 ? MS : 1][2];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
#pragma unroll
  for (int i = 0; i < (FP8 ? MS : 1); ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) blk[i][j] = f32x16{};

  // The MFMAs of step u; the loads of step ul, if any, are spread over them.
  // FP8: FRESH = u starts a scale block (its first MFMAs start from zero).
  auto compute = [&](int u, bool load, int ul, auto fresh_c) {
    constexpr bool FRESH = decltype(fresh_c)::value;
    const T* a_src = L.a[u % 3];
    const uint8_t* s_src = L.s[(u / sl) & 1];
    // lane (c32, h): k 32h .. 32h + 31 of its 2 columns (FP4 16 bytes, FP8 32)
    u32x4 bw[2][FP8 ? 2 : 1];
    float sc[2][2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int col = 64 * wn + 32 * nt + c32;
      const int ss = (col >> 3) & 1;
      if constexpr (FP8) {
        const uint8_t* bp = &L.b[u % 3][col * 64];
        bw[nt][0] = *reinterpret_cast<const u32x4*>(bp + 16 * ((2 * h) ^ b_swz(col)));
        bw[nt][1] = *reinterpret_cast<const u32x4*>(bp + 16 * ((2 * h + 1) ^ b_swz(col)));
      } else {
        // split: wave group wm takes half wm of K
        const uint8_t* bp = split ? &L.b[u % 3][col * 64 + 16 * ((2 * wm + h) ^ b_swz(col))]
                                  : &L.b[(u >> 1) & 1][col * 64 + 16 * ((2 * (u & 1) + h) ^ b_swz(col))];
        bw[nt][0] = *reinterpret_cast<const u32x4*>(bp);
        const int q = split ? wm : (u % kScaleSteps) >> 2;
        const uint32_t s2 = *reinterpret_cast<const uint16_t*>(
            &s_src[col * 32 + 16 * (q ^ ss) + 4 * (u & 3) + 2 * h]);
        sc[nt][0] = e4m3_to_f32<0>(s2);
        sc[nt][1] = e4m3_to_f32<1>(s2);
      }
    }
    // MFMA i takes k 32h + 8i .. 32h + 8i + 7 of both operands
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      V aop[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
        aop[ms] = *reinterpret_cast<const V*>(&a_src[lds_index(a_row0 + 32 * ms + c32, 4 * h + i)]);
      V bop[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        if constexpr (FP8)
          bop[nt] = Tr::decode8_fp8(bw[nt][i >> 1][2 * (i & 1)], bw[nt][i >> 1][2 * (i & 1) + 1]);
        else
          bop[nt] = Tr::decode8(bw[nt][0][i], Tr::make_scale(sc[nt][i >> 1]));
      }
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          if constexpr (FP8) {
            blk[ms][nt] = mfma32<T>(aop[ms], bop[nt], FRESH && i == 0 ? f32x16{} : blk[ms][nt]);
          } else {
            acc[ms][nt] = mfma32<T>(aop[ms], bop[nt], acc[ms][nt]);
          }
        }
      if (load) issue_part(ul, i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // FP8, after the last step of a scale block: running sum += block sum *
  // b_scale (FP32), column by column
  auto flush = [&](int u) {
    const uint8_t* s_src = L.s[(u / sl) & 1];
    const int idx = step_col(u) - slot_col(u / kScaleSteps);  // 0 .. 7
    float sc[2];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int col = 64 * wn + 32 * nt + c32;
      sc[nt] = *reinterpret_cast<const float*>(&s_src[col * 32 + 16 * ((idx >> 2) ^ ((col >> 3) & 1)) + 4 * (idx & 3)]);
    }
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ms][nt][r] = fmaf(blk[ms][nt][r], sc[nt], acc[ms][nt][r]);
  };
  // wait for everything but the n loads of the newest step, then barrier
  auto wait_all_but = [](int n) {
    switch (n) {
      case 2: wait_barrier<2>(); break;
      case 4: wait_barrier<4>(); break;
      case 6: wait_barrier<6>(); break;
      case 8: wait_barrier<8>(); break;
      case 10: wait_barrier<10>(); break;
      case 14: wait_barrier<14>(); break;
      default: wait_barrier<0>(); break;
    }
  };
  // one step: its next loads (FP8 issues them first; FP4 spreads them over
  // its MFMAs), its MFMAs, then the wait for the tiles of step u + 1
  auto step_body = [&](int u, auto fresh_c) {
    const bool ahead = u + 2 < nsteps;
    if (FP8 && ahead) issue(u + 2);
    compute(u, !FP8 && ahead, u + 2, fresh_c);
    if constexpr (FP8)
      if (u == nsteps - 1 || step_col(u + 1) != step_col(u)) flush(u);
    if (ahead)
      wait_all_but(loads_for(u + 2));  // the tiles of step u + 1 have landed
    else
      wait_barrier<0>();
  };


  issue(0);
  if (nsteps > 1) {
    issue(1);
    wait_all_but(loads_for(1));
  } else {
    wait_barrier<0>();
  }
  if constexpr (FP8) {
    // scale block by scale block: the first step of a block starts its sum
    // from zero, the last one flushes it (the last column also takes the
    // partial final block)
    for (int u0 = 0; u0 < nsteps;) {
      const int c = step_col(u0);
      const int end = c == cols - 1 ? nsteps : min(nsteps, (c + 1) * spb);
      step_body(u0, std::true_type{});
      for (int u = u0 + 1; u < end; ++u) step_body(u, std::false_type{});
      u0 = end;
    }
  } else {
    for (int u = 0; u < nsteps; ++u) step_body(u, std::false_type{});
  }

  // Epilogue: lane (c, h) holds columns 64 wn + 32 nt + c and rows
  // o_row0 + 32 ms + 8 (r / 4) + 4 h + r % 4 of the 128-row tile.
  // Y = acc * ws2 + bias, rounded once to T, is staged in LDS (the operand
  // stages are free now) and written back in whole 16-byte row pieces; tiles
  // on the ragged edge, or outputs that are not 16-byte aligned, store
  // element-wise.
  const int o_row0 = FP8 ? 64 * wm : 0;
  if (split) {
    // add the second half of K (wave group 1) to the first (wave group 0)
    float* red = reinterpret_cast<float*>(&L);
    if (wm == 1) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            red[(32 * ms + 8 * (r >> 2) + 4 * h + (r & 3)) * SC + 64 * wn + 32 * nt + c32] = acc[ms][nt][r];
    }
    __syncthreads();
    if (wm == 0) {
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            acc[ms][nt][r] += red[(32 * ms + 8 * (r >> 2) + 4 * h + (r & 3)) * SC + 64 * wn + 32 * nt + c32];
    }
    __syncthreads();
  }
  const float ws2 = FP8 ? 1.0f : *ws2p;
  constexpr int kOutPitch = SC + 8;  // elements per staged row (breaks bank aliasing)
  static_assert(sizeof(L) >= Sh::kTM * kOutPitch * sizeof(T), "output staging exceeds LDS");
  T* out = reinterpret_cast<T*>(&L);
  const bool wide = (N % 8 == 0) && (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && n0 + SC <= N;
  float bsum[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = min(n0 + 64 * wn + 32 * nt + c32, N - 1);
    bsum[nt] = bias ? static_cast<float>(bias[n]) : 0.0f;
  }
  if (!split || wm == 0) {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          out[(o_row0 + 32 * ms + 8 * (r >> 2) + 4 * h + (r & 3)) * kOutPitch + 64 * wn + 32 * nt + c32] =
              round_to<T>(fmaf(acc[ms][nt][r], ws2, bsum[nt]));
  }
  __syncthreads();
  if (wide) {
    // 128 rows x SC / 8 pieces of 16 bytes
#pragma unroll
    for (int i = 0; i < SC / 32; ++i) {
      const int q = tid + 512 * i;
      const int row = q / (SC / 8), piece = q % (SC / 8);
      if (row < rows_m)
        // non-temporal: Y is not read again here, keep A and B in the caches
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&out[row * kOutPitch + 8 * piece]),
                                    reinterpret_cast<u32x4*>(&Y[static_cast<size_t>(m0 + row) * N + n0 + 8 * piece]));
    }
  } else {
    for (int q = tid; q < 128 * SC; q += 512) {
      const int row = q / SC, col = q % SC;
      if (row < rows_m && n0 + col < N) Y[static_cast<size_t>(m0 + row) * N + n0 + col] = out[row * kOutPitch + col];
    }
  }
}

}  // namespace

template <typename T, bool FP8>
int launch_large(const MatmulArgs& a) {
  // Offsets inside the kernel are 32-bit and relative to the workgroup's
  // first row of A, B and the scales: 128 rows of A, 512 rows of B and of the
  // scales must each span less than 2^31 bytes (K < 2^22 covers all three).
  if (a.M > 0x7fffffff || a.N > 0x7fffffff || a.K >= (int64_t(1) << 22)) return -1;
  typedef LargeShape<FP8, false> Sh;
  const int64_t tiles_m = (a.M + Sh::kTM - 1) / Sh::kTM, tiles_n = (a.N + Sh::kTN - 1) / Sh::kTN;
  const int64_t ntiles = tiles_m * tiles_n;
  if (ntiles > 0x3fffffff) return -1;
  // The tiles of a last, partial round (at most half the CUs' worth) go to a
  // second launch that splits each of them over two workgroups, so that
  // round takes half as long (FP4, K % 128 == 0).
  const int64_t cus = device_cus(), rest = ntiles % cus;
  const bool split = !FP8 && a.K % (2 * BK) == 0 && rest > 0 && 2 * rest <= cus;
  const int64_t n_full = split ? ntiles - rest : ntiles;
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const T* A = static_cast<const T*>(a.A);
  const uint8_t* S = static_cast<const uint8_t*>(a.scales);
  const T* bias = static_cast<const T*>(a.bias);
  T* Y = static_cast<T*>(a.Y);
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int cols = static_cast<int>(a.scale_cols), bs = static_cast<int>(a.block_size);
  if (n_full > 0)
    hipLaunchKernelGGL((gemm_large_kernel<T, FP8, false>), dim3(static_cast<unsigned>(n_full)), dim3(512), 0, st, A,
                       a.B, S, a.ws2, bias, Y, M, N, K, cols, bs, static_cast<int>(tiles_m),
                       static_cast<int>(tiles_n), 0);
  if constexpr (!FP8) {
    if (split)
      hipLaunchKernelGGL((gemm_large_kernel<T, false, true>), dim3(static_cast<unsigned>(2 * rest)), dim3(512), 0,
                         st, A, a.B, S, a.ws2, bias, Y, M, N, K, cols, bs, static_cast<int>(tiles_m),
                         static_cast<int>(tiles_n), static_cast<int>(n_full));
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fp4_gemm(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_large<__bf16, false>(a) : launch_large<_Float16, false>(a);
}

int launch_fp8_gemm(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_large<__bf16, true>(a) : launch_large<_Float16, true>(a);
}

}  // namespace fp4w

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
// Two kernels (gfx950, wave64, 64 K per step, v_mfma_f32_32x32x16 with FP32
// accumulators):
//  * gemm_fp4_kernel: 4 waves per workgroup, one per SIMD, tile 256 x 256;
//    each wave holds all 256 rows and 64 columns (8 x 2 MFMA tiles) in 256
//    accumulation registers, so a decoded weight feeds 8 MFMA row tiles.
//    The E4M3 block scale is folded into the decoded BF16/FP16 operand, which
//    is exact (E2M1 x E4M3 needs 6 significand bits; [FP4 doc] §4);
//    weight_scale_2 and the bias are applied once in the epilogue.  The
//    tiles of a last, partial round are launched as 256 x 128 halves.  Up to
//    M = 128 the tiles are 128 rows high (4 MFMA row tiles per wave).
//  * gemm_fp8_kernel: 8 waves, tile 128 x 256, waves in a 2 (M) x 4 (N) grid,
//    each 64 x 64 = 2 x 2 MFMA tiles.  E4M3 -> T is exact; the FP32 block
//    scale is not representable in the operand, so every scale block
//    (block_size % 64 == 0) accumulates in a fresh set of FP32 accumulators,
//    which is then added to the running sum multiplied by its b_scale in FP32
//    ([FP8 doc] §2: B_dq = e4m3 * b_scale).  The two sets take 128 registers
//    per lane, which is why an FP8 wave holds half the outputs of an FP4 one.
//    A step's last MFMA group issues after the barrier that ends it, beside
//    the next step's first operand reads.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"
// [Blog]    = "ONNX Runtime #32128 - Why Dequantizing 4-Bit Weights Became the
//             Most Expensive Kernel in H200 Prefill"

#include <hip/hip_runtime.h>

#include <cstddef>
#include <type_traits>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr int BK = 64;
constexpr int kLdsRow = BK;     // elements per LDS row (no padding: XOR swizzle)
constexpr int kScaleSteps = 8;  // steps per scale slot

// 16-byte chunk c of row r sits in slot c ^ ((r >> 1) & 7): the 16 rows read
// by a 16-lane group at one logical chunk land in 16 distinct 16-byte slots of
// a 256-byte LDS line (rows are 128 bytes), so ds_read_b128 is conflict free.
__device__ __forceinline__ int lds_swz(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int lds_index(int row, int chunk) {
  return row * kLdsRow + ((chunk ^ lds_swz(row)) << 3);
}
// weight piece p (16 bytes) of column c sits in slot p ^ ((c >> 2) & 3)
__device__ __forceinline__ int b_swz(int col) { return (col >> 2) & 3; }

// Common structure of both kernels.
//  * Every operand tile moves global -> LDS by direct loads (no registers),
//    in the largest contiguous pieces its layout allows: an L2 request
//    carries one piece of at most 64 bytes of a line, so a 4-byte piece costs
//    as much as a full one (measured on the first version of this kernel).
//     - activations: ring of 3 one-step stages [rows][64] of T (rows of 128
//       contiguous bytes);
//     - FP4 weights: ring of 2 slots of two steps each, 64 contiguous bytes
//       per column; FP8 weights: ring of 3 one-step stages, 64 bytes per
//       column;
//     - scales: ring of 2 slots of eight steps each, 32 contiguous bytes per
//       column (32 E4M3 bytes, or 8 FP32 block scales starting at the first
//       block of the slot).
//    Every load goes through a buffer descriptor (32-bit offsets) whose base
//    is the workgroup's first row of A and first column of B and of the
//    scales, so any matrix size works; pieces past the matrix read zeros.
//    The per-step advance of the activation and weight loads is a scalar
//    offset and the LDS destination is wave-uniform, so issuing a load costs
//    no vector ALU work.
//  * The tiles of step t + 2 are requested during step t (FP8: at its start;
//    FP4: weights and scales at its start, the activation loads one per 8
//    MFMAs, the last quarter of them just after the barrier that ends step
//    t).  The only wait is, at the end of each step, for the tiles of step
//    t + 1 (loads complete in order; the loads of step t + 2 that are issued
//    first, FP4's weights and scales and FP8's scales, complete too, so that
//    the count is the same every step), then one barrier.  A slot is refilled only after the barrier that ends
//    its last reader's step.  The FP4 step loop is unrolled six steps at a
//    time (activation stage and weight-slot parity become constants) and
//    its last two steps, which issue no loads, are peeled off: each issued
//    instruction costs a wave with its SIMD to itself issue cycles that the
//    matrix pipe then waits for.
//  * LDS layouts are XOR-swizzled in 16-byte pieces (applied on the global
//    side, since one direct load writes its 64 lanes' data contiguously), so
//    the operand reads of a 16-lane group hit distinct banks.
//  * Lane (c, h) takes column c of each 32-wide N tile and k 32h .. 32h + 31
//    of each step for both operands (FP4: two 16-element scale blocks, one
//    16-byte LDS read); MFMA group i of the step takes k 32h + 8i .. + 7.
//    The operands of group i + 1 are read and decoded while the MFMAs of
//    group i issue.
//  * Tile order: workgroups are dispatched round-robin over the 8 XCDs, each
//    with its own L2, so the workgroup index is remapped to give every XCD a
//    contiguous range of tiles, walked in groups of tile rows.

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
// direct 16-byte buffer -> LDS load with a per-lane and a scalar offset; the
// range check is only guaranteed to see the per-lane offset
__device__ __forceinline__ void lds_load16_so(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(lds), 16, voff, soff, 0, 0);
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// tile (row, column) of tile index t in the order described above
__device__ __forceinline__ void tile_of(int t, int tiles_m, int tiles_n, int gm, int& tm, int& tn) {
  const int per_group = gm * tiles_n;
  const int first_m = (t / per_group) * gm;
  const int gsize = min(tiles_m - first_m, gm);
  tm = first_m + (t % per_group) % gsize;
  tn = (t % per_group) / gsize;
}

// Write back a ROWS x COLS output tile staged in LDS (`out`, rows of `pitch`
// elements): whole 16-byte row pieces where the tile lies inside N and Y is
// aligned, else element by element.
template <typename T, int THREADS, int ROWS, int COLS>
__device__ __forceinline__ void store_tile(const T* out, int pitch, T* Y, int m0, int n0, int rows_m, int N) {
  const bool wide = (N % 8 == 0) && (reinterpret_cast<uintptr_t>(Y) % 16 == 0) && n0 + COLS <= N;
  const int tid = threadIdx.x;
  if (wide) {
#pragma unroll
    for (int i = 0; i < ROWS * COLS / 8 / THREADS; ++i) {
      const int q = tid + THREADS * i;
      const int row = q / (COLS / 8), piece = q % (COLS / 8);
      if (row < rows_m)
        // non-temporal: Y is not read again here, keep A and B in the caches
        __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(&out[row * pitch + 8 * piece]),
                                    reinterpret_cast<u32x4*>(&Y[static_cast<size_t>(m0 + row) * N + n0 + 8 * piece]));
    }
  } else {
    for (int q = tid; q < ROWS * COLS; q += THREADS) {
      const int row = q / COLS, col = q % COLS;
      if (row < rows_m && n0 + col < N) Y[static_cast<size_t>(m0 + row) * N + n0 + col] = out[row * pitch + col];
    }
  }
}

// ------------------------------------------------------------------ FP4

template <int NT, int MS>
struct F4Shape {
  static constexpr int kTM = 32 * MS, kTN = 128 * NT;  // tile (NT = 1: half of a 256-column tile)
  static constexpr int kMS = MS;                       // MFMA row tiles per wave
  static constexpr int kAL = MS;                       // activation loads per wave and step
  static constexpr int kBL = 2 * NT;               // weight loads per wave and slot (two steps)
  static constexpr int kSL = 4 * NT;               // scale loads per wave and slot (eight steps)
  static constexpr int kGM = 4;                    // tile rows per group of the tile order
};

template <typename T, int NT, int MS>
struct F4Lds {
  uint8_t b[2][128 * NT * 64];  // 2 slots of two steps
  uint8_t s[2][128 * NT * 32];  // 2 slots of eight steps
  T a[3][32 * MS * kLdsRow];    // 3 x 32 KiB (MS = 8)
};

template <typename T, int NT, int MS_>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void gemm_fp4_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const uint8_t* __restrict__ scales,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int M, int N, int K, int cols,
    int tiles_m, int tiles_n, int t_first) {
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  typedef F4Shape<NT, MS_> Sh;
  typedef F4Lds<T, NT, MS_> Lds;
  __shared__ __attribute__((aligned(16))) Lds L;
  constexpr int MS = Sh::kMS, TN = Sh::kTN;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);

  // whole tiles: workgroup b takes tile b (contiguous ranges per XCD); halves
  // (tiles t_first ..): two workgroups per tile, 128 columns each
  int t = blockIdx.x;
  if (NT == 1)
    t = t_first + t / 2;
  else if (gridDim.x % 8 == 0)
    t = (t % 8) * (gridDim.x / 8) + t / 8;
  int tm, tn;
  tile_of(t, tiles_m, tiles_n, Sh::kGM, tm, tn);
  const int m0 = tm * Sh::kTM, n0 = tn * 256 + (NT == 1 ? 128 * (blockIdx.x & 1) : 0);
  const int rows_m = min(Sh::kTM, M - m0);     // activation rows of this tile
  const int rows_n = max(min(TN, N - n0), 0);  // weight / scale rows of this workgroup

  // Activations: instruction j of wave w writes stage rows 8q .. 8q + 7,
  // q = 4j + w; lane l lands in row 8q + l / 8, LDS chunk l % 8, which holds
  // global chunk (l % 8) ^ lds_swz(row).  Rows past M repeat the last row
  // (their outputs are not stored).  Byte offsets relative to row m0.
  uint32_t a_off[Sh::kAL];
#pragma unroll
  for (int j = 0; j < Sh::kAL; ++j) {
    const int row = 8 * (4 * j + wave) + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_swz(row);
    a_off[j] = 2u * static_cast<uint32_t>(min(row, rows_m - 1) * K + 8 * chunk);
  }
  const rsrc_t a_rsrc = make_rsrc(A + static_cast<size_t>(m0) * K,
                                  static_cast<uint32_t>(rows_m) * static_cast<uint32_t>(K) * 2u);
  // Weights: slot of two steps, 64 bytes per column (pieces 0-1 = the even
  // step, 2-3 = the odd step); instruction j of wave w covers columns
  // 16q .. 16q + 15, q = 4j + w; lane l lands in column 16q + l / 4, LDS
  // piece l % 4, holding global piece (l % 4) ^ b_swz(col).
  const uint32_t b_row = static_cast<uint32_t>(K / 2);
  uint32_t b_off[Sh::kBL];
#pragma unroll
  for (int j = 0; j < Sh::kBL; ++j) {
    const int col = 16 * (4 * j + wave) + (lane >> 2);
    b_off[j] = static_cast<uint32_t>(col) * b_row + 16u * ((lane & 3) ^ b_swz(col));
  }
  const rsrc_t b_rsrc = make_rsrc(B + static_cast<size_t>(n0) * b_row, static_cast<uint32_t>(rows_n) * b_row);
  // Scales: slot of eight steps, 32 bytes per column; instruction j of wave w
  // (4-byte pieces) covers columns 8q .. 8q + 7, q = kSL w + j; lane l lands
  // in column 8q + l / 8, LDS piece (l % 8) / 4 (16-byte), holding global
  // piece ((l % 8) / 4) ^ ((col >> 3) & 1).
  const uint32_t s_row = static_cast<uint32_t>(cols);
  uint32_t s_off[Sh::kSL];
#pragma unroll
  for (int j = 0; j < Sh::kSL; ++j) {
    const int col = 8 * (Sh::kSL * wave + j) + (lane >> 3);
    const int d = lane & 7;
    s_off[j] = static_cast<uint32_t>(col) * s_row + 4u * (d & 3) + 16u * ((d >> 2) ^ ((col >> 3) & 1));
  }
  const rsrc_t s_rsrc = make_rsrc(scales + static_cast<size_t>(n0) * s_row, static_cast<uint32_t>(rows_n) * s_row);

  const int nsteps = K / BK;
  // The loads of step u into activation stage `st` (= u % 3).  Activation
  // and weight offsets stay in range at every step, and lanes past the
  // matrix are out of range on their per-lane offset alone, so the step's
  // advance can be the scalar offset.
  T* const a_lds = &L.a[0][0] + wave * 8 * kLdsRow;
  auto issue_a = [&](int st, int u, int j) {
    lds_load16_so(a_rsrc, a_lds + st * (32 * MS * kLdsRow) + 4 * j * 8 * kLdsRow, a_off[j],
                  static_cast<uint32_t>(u * BK * 2));
  };
  auto issue_b = [&](int u) {  // u even: the slot of steps u, u + 1
#pragma unroll
    for (int j = 0; j < Sh::kBL; ++j)
      lds_load16_so(b_rsrc, &L.b[(u >> 1) & 1][(4 * j + wave) * 1024], b_off[j], 32u * u);
  };
  auto issue_s = [&](int u) {  // u % 8 == 0: the slot of steps u .. u + 7
    const int c = u / kScaleSteps;
#pragma unroll
    for (int j = 0; j < Sh::kSL; ++j)
      buf_load_lds<4>(s_rsrc, s_off[j] + 32u * c, &L.s[c & 1][(Sh::kSL * wave + j) * 256]);
  };
  constexpr int kAG = Sh::kAL / 4;  // activation loads per MFMA group

  // lane (c32, h): column c32 of each 32-wide N tile, k half h of every step
  const int c32 = lane & 31, h = lane >> 5;
  f32x16 acc[MS][NT];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = f32x16{};

  // this lane's packed weights (16 bytes per column tile) and scales of a step
  u32x4 bw[NT];
  float sc[NT][2];
  // Per-lane LDS byte addresses of the operand reads.  Weight piece
  // (2 (u & 1) + h) ^ b_swz(col) of slot (u >> 1) & 1 and scale pair
  // (u % 8) / 4 ^ ((col >> 3) & 1), byte 4 (u & 3) + 2 h, of slot (u / 8) & 1
  // differ from the step-0 address only in bits that are zero there, so a
  // step's address is the step-0 address XOR a wave-uniform value.
  uint32_t b_rd[NT], s_rd[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = 32 * NT * wave + 32 * nt + c32;
    b_rd[nt] = static_cast<uint32_t>(offsetof(Lds, b)) + col * 64 + 16 * (h ^ b_swz(col));
    s_rd[nt] = static_cast<uint32_t>(offsetof(Lds, s)) + col * 32 + 16 * ((col >> 3) & 1) + 2 * h;
  }
  const char* lds_bytes = reinterpret_cast<const char*>(&L);
  // raw reads of step u's weights and scale bytes; set_b then makes them the
  // current step's (the scale decode waits for nothing by then)
  auto read_b = [&](int u, u32x4 (&w)[NT], uint32_t (&s2)[NT]) {
    const uint32_t ub = ((u & 1) << 5) | (((u >> 1) & 1) * sizeof(L.b[0]));
    const uint32_t us = (((u % kScaleSteps) >> 2) << 4) | ((u & 3) << 2) | (((u / kScaleSteps) & 1) * sizeof(L.s[0]));
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      w[nt] = *reinterpret_cast<const u32x4*>(lds_bytes + (b_rd[nt] ^ ub));
      s2[nt] = *reinterpret_cast<const uint16_t*>(lds_bytes + (s_rd[nt] ^ us));
    }
  };
  auto set_b = [&](const u32x4 (&w)[NT], const uint32_t (&s2)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bw[nt] = w[nt];
      sc[nt][0] = e4m3_to_f32<0>(s2[nt]);
      sc[nt][1] = e4m3_to_f32<1>(s2[nt]);
    }
  };
  // activation fragment of chunk 4 h + i, row c32 of row tile 0, stage 0
  uint32_t a_rd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_rd[i] = 2 * lds_index(c32, 4 * h + i);
  auto read_a = [&](int st, int i, V (&aop)[MS]) {
    const char* a_src = reinterpret_cast<const char*>(&L.a[0][0]) + st * (2 * 32 * MS * kLdsRow) + a_rd[i];
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) aop[ms] = *reinterpret_cast<const V*>(a_src + ms * (2 * 32 * kLdsRow));
  };
  auto dec_b = [&](int i, V (&bop)[NT]) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) bop[nt] = Tr::decode8(bw[nt][i], Tr::make_scale(sc[nt][i >> 1]));
  };
  auto mfmas = [&](const V (&aop)[MS], const V (&bop)[NT]) {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[ms][nt] = mfma32<T>(aop[ms], bop[nt], acc[ms][nt]);
  };
  // scheduling: per MFMA, one LDS read (first MS MFMAs) and a share of the
  // vector ALU work of the next group's operands; with LOADS, one activation
  // load per kMf / kAG MFMAs
  auto interleave = [](auto loads_c, auto reads_c) {
    constexpr bool LOADS = decltype(loads_c)::value;
    constexpr int kReads = MS + decltype(reads_c)::value;  // LDS reads of the group
    constexpr int kMf = MS * NT, kVa = 32 * NT / kMf + 1;
#pragma unroll
    for (int k = 0; k < kMf; ++k) {
      if (k < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, kVa, 0);            // vector ALU
      if (LOADS && k % (kMf / kAG) == 1) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // activation load
    }
  };

  V aop[MS], bop[NT];
  // One step u (activations in stage st = u % 3).  AHEAD: it issues the
  // loads of step u + 2 (weights and scales at its start, activations one
  // per kMf / kAG MFMAs, the last quarter after the barrier).  The MFMAs of
  // group i run while the operands of group i + 1 are read and decoded; the
  // last group's MFMAs run after the barrier that ends the step, together
  // with the first reads of step u + 1.
  auto step = [&](int u, int st, int par, auto ahead_c) {  // par: u & 1, or -1 (not known)
    constexpr bool AHEAD = decltype(ahead_c)::value;
    const int st1 = st == 2 ? 0 : st + 1;  // (u + 1) % 3
    const int st2 = st == 0 ? 2 : st - 1;  // (u + 2) % 3
    if (AHEAD) {
      if (par >= 0 ? par == 0 : ((u + 2) & 1) == 0) issue_b(u + 2);
      if ((u + 2) % kScaleSteps == 0) issue_s(u + 2);
    }
    // step u + 1's weights and scales are in LDS since the barrier that
    // ended step u - 1; they are read in group 1, long before their use
    u32x4 bwn[NT];
    uint32_t s2n[NT];
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      V an[MS], bn[NT];
      read_a(st, i + 1, an);
      if (i == 1) read_b(min(u + 1, nsteps - 1), bwn, s2n);
      dec_b(i + 1, bn);
      if (AHEAD) {
#pragma unroll
        for (int j = kAG * i; j < kAG * (i + 1); ++j) issue_a(st2, u + 2, j);
      }
      mfmas(aop, bop);
      if (i == 1)
        interleave(ahead_c, std::integral_constant<int, 2 * NT>{});
      else
        interleave(ahead_c, std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the next group's operand reads
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) aop[ms] = an[ms];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bop[nt] = bn[nt];
    }
    // The tiles of step u + 1 have landed once every wave passes this
    // barrier.  With AHEAD the loads of step u + 2 issued so far may stay in
    // flight except its weights and scales (issued first, a step ago).
    if (AHEAD)
      wait_barrier<3 * kAG>();
    else
      wait_barrier<0>();
    {
      V an[MS], bn[NT];
      set_b(bwn, s2n);                           // after the last step: unused
      read_a(u + 1 < nsteps ? st1 : st, 0, an);  // after the last step: re-read, unused
      dec_b(0, bn);
      if (AHEAD) {
#pragma unroll
        for (int j = 3 * kAG; j < 4 * kAG; ++j) issue_a(st2, u + 2, j);
      }
      mfmas(aop, bop);
      interleave(ahead_c, std::integral_constant<int, 0>{});
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the next group's operand reads
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) aop[ms] = an[ms];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bop[nt] = bn[nt];
    }
  };

  issue_b(0);
  issue_s(0);
#pragma unroll
  for (int j = 0; j < Sh::kAL; ++j) issue_a(0, 0, j);
  if (nsteps > 1) {
    // step 1's weights share slot 0 with step 0's
#pragma unroll
    for (int j = 0; j < Sh::kAL; ++j) issue_a(1, 1, j);
    wait_barrier<Sh::kAL>();
  } else {
    wait_barrier<0>();
  }
  {
    u32x4 w[NT];
    uint32_t s2[NT];
    read_b(0, w, s2);
    set_b(w, s2);
  }
  read_a(0, 0, aop);
  dec_b(0, bop);
  int u = 0, st = 0;
  // six steps at a time (activation stage u % 3 and weight slot parity are
  // then constants), then the rest one by one
  for (; u + 7 < nsteps; u += 6) {
    step(u, 0, 0, std::true_type{});
    step(u + 1, 1, 1, std::true_type{});
    step(u + 2, 2, 0, std::true_type{});
    step(u + 3, 0, 1, std::true_type{});
    step(u + 4, 1, 0, std::true_type{});
    step(u + 5, 2, 1, std::true_type{});
  }
  for (; u + 2 < nsteps; ++u) {
    step(u, st, -1, std::true_type{});
    st = st == 2 ? 0 : st + 1;
  }
  for (; u < nsteps; ++u) {
    step(u, st, -1, std::false_type{});
    st = st == 2 ? 0 : st + 1;
  }

  // Epilogue: lane (c, h) holds columns 32 NT wave + 32 nt + c and rows
  // 32 ms + 8 (r / 4) + 4 h + r % 4 of the tile.  Y = acc * ws2 + bias,
  // rounded once to T, is staged in LDS (the operand rings, free once every
  // wave has passed the barrier below and its last loads have landed).
  wait_barrier<0>();
  const float ws2 = *ws2p;
  constexpr int kOutPitch = TN + 8;  // elements per staged row (breaks bank aliasing)
  static_assert(sizeof(L) >= Sh::kTM * kOutPitch * sizeof(T), "output staging exceeds LDS");
  T* out = reinterpret_cast<T*>(&L);
  float bsum[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int n = min(n0 + 32 * NT * wave + 32 * nt + c32, N - 1);
    bsum[nt] = bias ? static_cast<float>(bias[n]) : 0.0f;
  }
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        out[(32 * ms + 8 * (r >> 2) + 4 * h + (r & 3)) * kOutPitch + 32 * NT * wave + 32 * nt + c32] =
            round_to<T>(fmaf(acc[ms][nt][r], ws2, bsum[nt]));
  __syncthreads();
  store_tile<T, 256, Sh::kTM, TN>(out, kOutPitch, Y, m0, n0, rows_m, N);
}

// ------------------------------------------------------------------ FP8

struct F8Shape {
  static constexpr int kTM = 128, kTN = 256;  // tile
  static constexpr int kWaveM = 64;           // output rows of a wave
  static constexpr int kMS = kWaveM / 32;     // MFMA row tiles of a wave
  static constexpr int kAL = 2;               // activation loads per wave and step
  static constexpr int kBL = 2;               // weight loads per wave and step
  static constexpr int kSL = 4;               // scale loads per wave and slot
  static constexpr int kGM = 4;               // tile rows per group of the tile order
};

template <typename T>
struct F8Lds {
  T a[3][128 * kLdsRow];   // 3 x 16 KiB
  uint8_t b[3][256 * 64];  // 3 one-step stages
  uint8_t s[2][256 * 32];  // 2 slots of eight steps
};

template <typename T>
__global__ __launch_bounds__(512) void gemm_fp8_kernel(const T* __restrict__ A, const uint8_t* __restrict__ B,
                                                       const uint8_t* __restrict__ scales, const T* __restrict__ bias,
                                                       T* __restrict__ Y, int M, int N, int K, int cols, int bs,
                                                       int tiles_m, int tiles_n) {
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  typedef F8Shape Sh;
  __shared__ __attribute__((aligned(16))) F8Lds<T> L;
  constexpr int MS = Sh::kMS;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = uniform(tid >> 6);
  // wave group wm takes rows 64 wm .. 64 wm + 63, wn columns 64 wn .. + 63
  const int wm = wave >> 2, wn = wave & 3;

  int t = blockIdx.x;
  if (gridDim.x % 8 == 0) t = (t % 8) * (gridDim.x / 8) + t / 8;
  int tm, tn;
  tile_of(t, tiles_m, tiles_n, Sh::kGM, tm, tn);
  const int m0 = tm * Sh::kTM, n0 = tn * Sh::kTN;
  const int rows_m = min(Sh::kTM, M - m0);
  const int rows_n = max(min(Sh::kTN, N - n0), 0);

  // activations: instruction j of wave w writes rows 8q .. 8q + 7, q = 8j + w
  // (lane layout and swizzle as in the FP4 kernel)
  uint32_t a_off[Sh::kAL];
#pragma unroll
  for (int j = 0; j < Sh::kAL; ++j) {
    const int row = 8 * (8 * j + wave) + (lane >> 3);
    const int chunk = (lane & 7) ^ lds_swz(row);
    a_off[j] = 2u * static_cast<uint32_t>(min(row, rows_m - 1) * K + 8 * chunk);
  }
  const rsrc_t a_rsrc = make_rsrc(A + static_cast<size_t>(m0) * K,
                                  static_cast<uint32_t>(rows_m) * static_cast<uint32_t>(K) * 2u);
  // weights: one-step stage, 64 bytes per column; instruction j of wave w
  // covers columns 16q .. 16q + 15, q = 8j + w
  const uint32_t b_row = static_cast<uint32_t>(K);
  uint32_t b_off[Sh::kBL];
#pragma unroll
  for (int j = 0; j < Sh::kBL; ++j) {
    const int col = 16 * (8 * j + wave) + (lane >> 2);
    b_off[j] = static_cast<uint32_t>(col) * b_row + 16u * ((lane & 3) ^ b_swz(col));
  }
  const rsrc_t b_rsrc = make_rsrc(B + static_cast<size_t>(n0) * b_row, static_cast<uint32_t>(rows_n) * b_row);
  // scales: slot of eight FP32 block scales starting at the block of the
  // slot's first step, 32 bytes per column; instruction j of wave w covers
  // columns 8q .. 8q + 7, q = kSL w + j
  const uint32_t s_row = static_cast<uint32_t>(cols) * 4u;
  uint32_t s_off[Sh::kSL];
#pragma unroll
  for (int j = 0; j < Sh::kSL; ++j) {
    const int col = 8 * (Sh::kSL * wave + j) + (lane >> 3);
    const int d = lane & 7;
    s_off[j] = static_cast<uint32_t>(col) * s_row + 4u * (d & 3) + 16u * ((d >> 2) ^ ((col >> 3) & 1));
  }
  const rsrc_t s_rsrc = make_rsrc(scales + static_cast<size_t>(n0) * s_row, static_cast<uint32_t>(rows_n) * s_row);
  const int spb = bs / BK;  // steps per scale block (block_size % 64 == 0)
  // the first scale column of the slot holding steps 8c .. 8c + 7
  auto slot_col = [&](int c) {
    return min(static_cast<int>(static_cast<uint32_t>(kScaleSteps * c) / static_cast<uint32_t>(spb)), cols - 1);
  };

  const int nsteps = K / BK;
  int slot_first0 = 0, slot_first1 = 0;  // first scale column of scale slots 0 and 1, set when loaded
  // The loads of step u into stage st (= u % 3): the scale slot first (every
  // eighth step), then activations and weights, so that waiting until only
  // those of the last issued step are in flight (a count that is the same
  // every step) also covers its scales, issued a step earlier.
  auto issue = [&](int u, int st) {
    const uint32_t step = static_cast<uint32_t>(u * BK);
    if (u % kScaleSteps == 0) {
      const int c = u / kScaleSteps;
      const int first = slot_col(c);
      if (c & 1)
        slot_first1 = first;
      else
        slot_first0 = first;
      const uint32_t base = 4u * static_cast<uint32_t>(first);
#pragma unroll
      for (int j = 0; j < Sh::kSL; ++j)
        buf_load_lds<4>(s_rsrc, s_off[j] + base, &L.s[c & 1][(Sh::kSL * wave + j) * 256]);
    }
#pragma unroll
    for (int j = 0; j < Sh::kAL; ++j)
      lds_load16_so(a_rsrc, &L.a[st][(8 * j + wave) * 8 * kLdsRow], a_off[j], 2u * step);
#pragma unroll
    for (int j = 0; j < Sh::kBL; ++j) lds_load16_so(b_rsrc, &L.b[st][(8 * j + wave) * 1024], b_off[j], step);
  };
  constexpr int kStepLoads = Sh::kAL + Sh::kBL;

  const int c32 = lane & 31, h = lane >> 5;
  const int a_row0 = Sh::kWaveM * wm;  // this wave's first row in an activation stage
  f32x16 acc[MS][2];
  f32x16 blk[MS][2];  // the current scale block's sum (fresh at the first step of a block)
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = f32x16{};
      blk[i][j] = f32x16{};
    }
  // per-lane LDS byte offsets of the operand reads within a stage:
  // activation chunk 4h + i of row a_row0 + c32 (row tile ms adds 32 rows),
  // weight pieces 2h and 2h + 1 of column 64 wn + 32 nt + c32
  uint32_t a_rd[4], b_rd[2][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) a_rd[i] = 2u * static_cast<uint32_t>(lds_index(a_row0 + c32, 4 * h + i));
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int col = 64 * wn + 32 * nt + c32;
#pragma unroll
    for (int p = 0; p < 2; ++p) b_rd[nt][p] = static_cast<uint32_t>(col * 64 + 16 * ((2 * h + p) ^ b_swz(col)));
  }

  // Operands carried from step to step: the raw weights of the current step
  // (bw) and the decoded operands of its first MFMA group (aop, bop).  They
  // are read after the barrier that ends the previous step, beside that
  // step's last MFMA group, so a step never starts by waiting for LDS.
  // Lane (c32, h) takes k 32h .. 32h + 31 of its 2 columns (32 bytes).
  u32x4 bw[2][2];
  V aop[MS], bop[2];
  auto stage_a = [&](int st) { return reinterpret_cast<const char*>(&L.a[0][0]) + st * sizeof(L.a[0]); };
  auto read_a = [&](const char* a_src, int i, V (&o)[MS]) {
#pragma unroll
    for (int ms = 0; ms < MS; ++ms) o[ms] = *reinterpret_cast<const V*>(a_src + a_rd[i] + ms * (2 * 32 * kLdsRow));
  };
  auto read_bw = [&](int st) {
    const char* b_src = reinterpret_cast<const char*>(&L.b[0][0]) + st * sizeof(L.b[0]);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int p = 0; p < 2; ++p) bw[nt][p] = *reinterpret_cast<const u32x4*>(b_src + b_rd[nt][p]);
  };
  auto dec_b = [&](int i, V (&o)[2]) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) o[nt] = Tr::decode8_fp8(bw[nt][i >> 1][2 * (i & 1)], bw[nt][i >> 1][2 * (i & 1) + 1]);
  };
  // after the last step u of the block with scale column c: running sum +=
  // block sum * b_scale (FP32), column by column
  auto flush = [&](int u, int c) {
    const uint8_t* s_src = L.s[(u / kScaleSteps) & 1];
    const int idx = c - ((u / kScaleSteps) & 1 ? slot_first1 : slot_first0);  // 0 .. 7
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
  // One step u (stage st) of the block with scale column c ending before
  // step `end`: its loads of step u + 2; MFMA groups 0 - 2, each beside the
  // reads and decode of the next group's operands (group 0 starts a block's
  // sum from zero); the barrier after which the tiles of step u + 1 have
  // landed and no wave reads stage st any more; group 3 beside the reads of
  // step u + 1's first operands (after the last step: re-reads, unused);
  // after the block's last step its flush.
  auto step_body = [&](int u, int st, int c, int end, auto fresh_c) {
    constexpr bool FRESH = decltype(fresh_c)::value;
    const bool ahead = u + 2 < nsteps;
    if (ahead) issue(u + 2, st == 0 ? 2 : st - 1);
    const char* a_src = stage_a(st);
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      V an[MS], bn[2];
      read_a(a_src, i + 1, an);
      dec_b(i + 1, bn);
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          blk[ms][nt] = mfma32<T>(aop[ms], bop[nt], FRESH && i == 0 ? f32x16{} : blk[ms][nt]);
      // per MFMA: one LDS read (first MS MFMAs), then a share of the next
      // group's decode
#pragma unroll
      for (int k = 0; k < 2 * MS; ++k) {
        if (k < MS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);              // vector ALU
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) aop[ms] = an[ms];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) bop[nt] = bn[nt];
    }
    if (ahead)
      wait_barrier<kStepLoads>();
    else
      wait_barrier<0>();
    {
      V a3[MS], b3[2];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) a3[ms] = aop[ms];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) b3[nt] = bop[nt];
      const int st1 = st == 2 ? 0 : st + 1;
      read_bw(st1);
      read_a(stage_a(st1), 0, aop);
      dec_b(0, bop);
#pragma unroll
      for (int ms = 0; ms < MS; ++ms)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) blk[ms][nt] = mfma32<T>(a3[ms], b3[nt], blk[ms][nt]);
      // per MFMA: some of the next step's six operand reads (three beside
      // the first), and from the third on a share of its first decode
#pragma unroll
      for (int k = 0; k < 2 * MS; ++k) {
        if (k == 0)
          __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // LDS read
        else
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
        if (k >= 2) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);  // vector ALU
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (u == end - 1) flush(u, c);
  };

  issue(0, 0);
  if (nsteps > 1) {
    issue(1, 1);
    wait_barrier<kStepLoads>();
  } else {
    wait_barrier<0>();
  }
  read_bw(0);
  read_a(stage_a(0), 0, aop);
  dec_b(0, bop);
  // scale block by scale block: the first step of a block starts its sum
  // from zero, the last one flushes it (the last column also takes the
  // partial final block); st is the stage of step u, u % 3
  int st = 0;
  for (int u0 = 0, c = 0; u0 < nsteps; ++c) {  // block c starts at step c * spb
    const int end = c == cols - 1 ? nsteps : min(nsteps, (c + 1) * spb);
    step_body(u0, st, c, end, std::true_type{});
    st = st == 2 ? 0 : st + 1;
    for (int u = u0 + 1; u < end; ++u) {
      step_body(u, st, c, end, std::false_type{});
      st = st == 2 ? 0 : st + 1;
    }
    u0 = end;
  }

  // Epilogue: lane (c, h) holds columns 64 wn + 32 nt + c and rows
  // 64 wm + 32 ms + 8 (r / 4) + 4 h + r % 4 of the tile; after a barrier
  // that follows every wave's last LDS reads, the operand rings are free.
  __syncthreads();
  constexpr int kOutPitch = Sh::kTN + 8;
  static_assert(sizeof(L) >= Sh::kTM * kOutPitch * sizeof(T), "output staging exceeds LDS");
  T* out = reinterpret_cast<T*>(&L);
  float bsum[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    const int n = min(n0 + 64 * wn + 32 * nt + c32, N - 1);
    bsum[nt] = bias ? static_cast<float>(bias[n]) : 0.0f;
  }
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        out[(a_row0 + 32 * ms + 8 * (r >> 2) + 4 * h + (r & 3)) * kOutPitch + 64 * wn + 32 * nt + c32] =
            round_to<T>(acc[ms][nt][r] + bsum[nt]);
  __syncthreads();
  store_tile<T, 512, Sh::kTM, Sh::kTN>(out, kOutPitch, Y, m0, n0, rows_m, N);
}

}  // namespace

// Offsets inside the kernels are 32-bit and relative to the workgroup's
// first row of A, B and the scales: 256 rows of A, 256 rows of B and of the
// scales must each span less than 2^31 bytes (K < 2^22 covers all three).
template <typename T, int MS>
int launch_fp4_ms(const MatmulArgs& a) {
  constexpr int TM = 32 * MS;
  const int64_t tiles_m = (a.M + TM - 1) / TM, tiles_n = (a.N + 255) / 256;
  const int64_t ntiles = tiles_m * tiles_n;
  if (ntiles > 0x3fffffff) return -1;
  // The tiles of a last, partial round (at most half the CUs' worth) go to a
  // second launch as two TM x 128 halves each, so that round takes about
  // half as long.
  const int64_t cus = device_cus(), rest = ntiles % cus;
  const bool halves = rest > 0 && 2 * rest <= cus;
  const int64_t n_full = halves ? ntiles - rest : ntiles;
  const hipStream_t st = static_cast<hipStream_t>(a.stream);
  const T* A = static_cast<const T*>(a.A);
  const uint8_t* S = static_cast<const uint8_t*>(a.scales);
  const T* bias = static_cast<const T*>(a.bias);
  T* Y = static_cast<T*>(a.Y);
  const int M = static_cast<int>(a.M), N = static_cast<int>(a.N), K = static_cast<int>(a.K);
  const int cols = static_cast<int>(a.scale_cols);
  if (n_full > 0)
    hipLaunchKernelGGL((gemm_fp4_kernel<T, 2, MS>), dim3(static_cast<unsigned>(n_full)), dim3(256), 0, st, A, a.B,
                       S, a.ws2, bias, Y, M, N, K, cols, static_cast<int>(tiles_m), static_cast<int>(tiles_n), 0);
  if (halves)
    hipLaunchKernelGGL((gemm_fp4_kernel<T, 1, MS>), dim3(static_cast<unsigned>(2 * rest)), dim3(256), 0, st, A, a.B,
                       S, a.ws2, bias, Y, M, N, K, cols, static_cast<int>(tiles_m), static_cast<int>(tiles_n),
                       static_cast<int>(n_full));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// 256-row tiles (8 MFMA row tiles per wave); up to 128 rows, 128-row tiles,
// which halve a prompt chunk's padding and per-workgroup work
template <typename T>
int launch_fp4(const MatmulArgs& a) {
  if (a.M > 0x7fffffff || a.N > 0x7fffffff || a.K >= (int64_t(1) << 22)) return -1;
  return a.M <= 128 ? launch_fp4_ms<T, 4>(a) : launch_fp4_ms<T, 8>(a);
}

template <typename T>
int launch_fp8(const MatmulArgs& a) {
  if (a.M > 0x7fffffff || a.N > 0x7fffffff || a.K >= (int64_t(1) << 22)) return -1;
  const int64_t tiles_m = (a.M + 127) / 128, tiles_n = (a.N + 255) / 256;
  const int64_t ntiles = tiles_m * tiles_n;
  if (ntiles > 0x3fffffff) return -1;
  hipLaunchKernelGGL((gemm_fp8_kernel<T>), dim3(static_cast<unsigned>(ntiles)), dim3(512), 0,
                     static_cast<hipStream_t>(a.stream), static_cast<const T*>(a.A), a.B,
                     static_cast<const uint8_t*>(a.scales), static_cast<const T*>(a.bias), static_cast<T*>(a.Y),
                     static_cast<int>(a.M), static_cast<int>(a.N), static_cast<int>(a.K),
                     static_cast<int>(a.scale_cols), static_cast<int>(a.block_size), static_cast<int>(tiles_m),
                     static_cast<int>(tiles_n));
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_fp4_gemm(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_fp4<__bf16>(a) : launch_fp4<_Float16>(a);
}

int launch_fp8_gemm(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_fp8<__bf16>(a) : launch_fp8<_Float16>(a);
}

}  // namespace fp4w

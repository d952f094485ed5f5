// Decode GEMV (1 <= M <= 8) for weight-only FP4 and FP8, on MFMA.
//
// Memory-bound: every packed weight byte and scale byte is read from HBM once,
// in whole 128-byte lines; activations (M x K, at most a few hundred KiB) come
// from LDS or L2.
//
// Common structure (the pages' CUDA version is [FP4 doc] §4 "Tensor-core
// sub-path" / [FP8 doc] §4.1, with mma.m16n8k16; this is re-derived for the
// CDNA4 MFMA layouts).  A wave owns a tile of 16 output columns n (the MFMA B
// operand: lane l supplies column l % 16).  K is a reduction axis, so it is
// permuted freely as long as both operands agree: in window w (128 k) lane
// group g = l / 16 takes the contiguous chunk c = 4w + g of 32 k of its
// column, one 16-byte fragment per lane for FP4 (two for FP8).
//
// FP4 (16x16x32 MFMA, "block-diagonal" activations).  Folding the E4M3 scale
// into BF16 weights would be exact ([FP4 doc] §4), but costs a convert, two
// FP32 multiplies and a pack per pair of weights, which makes a wave64 GEMV
// VALU-bound on CDNA4.  Instead the weights are converted unscaled (one
// instruction per pair) and every 16-k scale block gets its own FP32 dot,
// scaled by its E4M3 value with one FMA.  Four blocks share each MFMA: lane
// group g holds blocks 2g and 2g + 1 of the window, so in MFMA (s, p) the
// four lane groups supply piece p (8 k) of blocks 2g + s, g = 0..3.  For
// M <= 4, row i = 4 m' + q of the A operand carries activation row m' in the
// k slots of lane group q only, and zeros elsewhere; summing the two pieces
// p therefore leaves in result row (m', q) the full dot of row m' with block
// 2q + s.  The result lane (column n, group g) holds rows 4g .. 4g + 3 = the
// four blocks of one activation row, so a window costs 4 MFMAs and 8 FMAs,
// with no data exchange between lanes.  weight_scale_2 and the bias are
// applied once in the epilogue.
//
// FP4 with 5 <= M <= 8 ("row pairs").  Four activation rows per MFMA would
// take two sets of MFMAs per window, each a quarter useful.  Instead, in MFMA
// t (t = 0 .. 3) lane groups 0 and 1 supply the two 8-k pieces of block t of
// the window and groups 2 and 3 those of block 4 + t, so a block's 16 k
// meet in one MFMA; row i = 2m + h of the A operand carries activation row m
// in the k slots of half h (groups 2h, 2h + 1) only.  Result row 2m + h is
// then the dot of row m with block 4h + t, and the lane (n, g) holds rows
// 2g and 2g + 1, each with two blocks: a window costs 4 MFMAs (half useful)
// and 16 FMAs.  Lane group g's weights are piece g & 1 of four blocks, two
// dwords from each of two 16-byte chunks (two ds_read2_b32).
//
// FP8 (16x16x32 MFMA).  E4M3 -> T is exact and the FP32 block scale is
// applied to a window (128 k, inside one scale block: block_size % 128 == 0)
// accumulated in a fresh MFMA accumulator.  Result lane (n, g) holds rows
// 4g .. 4g + 3.
//
// Pipeline: a wave keeps D units of weights (below) in flight ahead of the one
// it multiplies; the pipeline runs as one flat sequence over all tile groups
// the (persistent) workgroup owns, so it never drains between tiles.  All
// loads are raw buffer loads and branch-free (tails read zeros), so the loop
// only ever waits for its oldest loads.  A workgroup is KS x TPW waves: KS
// waves split the K windows of one tile (the page's KSplit, reduced through
// LDS), TPW tiles side by side.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"

#include <hip/hip_runtime.h>

#include <mutex>

#include "device.h"
#include "launch.h"
#include "nvfp4_block.h"

namespace fp4w {
namespace {

constexpr int kWaves = 8;  // waves per workgroup (KS x TPW)

// Weights travel global -> LDS by direct loads (no registers).  A unit (FP4:
// two 128-k windows, FP8: one) is 128 contiguous bytes of each of the wave's
// 16 rows, fetched by two instructions of 8 rows x 128 bytes.  HBM streams at
// full rate only when an instruction requests whole 128-byte lines; 16 rows
// x 64 bytes per instruction (half lines) reaches about two thirds of it.
// Each row's eight 16-byte chunks are loaded by 8 adjacent lanes in the order
// chunk ^ (row & 7), so the LDS copy comes out XOR-swizzled and the fragment
// reads (lane (li, g): one chunk of row li) are free of bank conflicts.  A
// wave has a private ring of D + 1 unit slots of 2 KiB and waits for its own
// loads only, with no barrier.
constexpr uint32_t kUnitBytes = 2048;  // one unit slot: 16 rows x 128 bytes
constexpr int kSlicePitch = 144;       // FP4 scale slice: bytes per row (128 + 16 against bank conflicts)

template <bool FP8>
constexpr uint32_t slice_bytes() {
  return 16u * kSlicePitch;  // FP4: 128 E4M3 bytes per row, FP8: 32 FP32 scales per row
}

// Units per scale piece.  FP4: 8 E4M3 bytes per window, 128 bytes per row =
// 16 windows = 8 units, loaded like the weights (8 rows x 128 bytes per
// instruction).  FP8: one FP32 scale per 64-k half window at most
// (block_size % 64 == 0), 32 scales of a row = 128 bytes per piece of 16
// windows.
template <bool FP8>
constexpr int kScaleUnits = FP8 ? 16 : 8;

// Activations streamed from L2 (ACT_REG): each unit brings the activation
// bytes of its K range, row-major (rows of 512 bytes for FP4's two windows,
// 256 bytes for FP8's one), so that every load instruction requests whole
// lines: FP4 2R instructions of 2 rows, FP8 two of 4 rows.  The multiply
// stores them in a wave-private LDS staging area and reads them back in the
// MFMA layout.
template <bool FP8, int R>
constexpr int kActLoads = FP8 ? 2 : 2 * R;
constexpr uint32_t kStagePitch4 = 528;  // FP4: bytes per staged row (512 + 16)
constexpr uint32_t kStagePitch8 = 272;  // FP8: bytes per staged row (256 + 16)

// Staging bytes per wave: FP4 4R rows and a 128-byte zero block for the
// lanes that carry no row; FP8 8 rows.
template <bool FP8, int R>
constexpr uint32_t stage_bytes() {
  return FP8 ? 8u * kStagePitch8 : 4u * R * kStagePitch4 + 128u;
}

// Register part of one unit for one lane: the scale piece (first unit of
// each piece), the bias bits of the lane's column (first unit of a tile) and,
// when they come from L2 (ACT_REG), the activations.
template <bool FP8, bool ACT_REG, int R>
struct Raw;
template <bool ACT_REG, int R>
struct Raw<false, ACT_REG, R> {
  u32x4 sc[2];      // rows lr and 8 + lr, 16 bytes each from a dword-aligned offset
  uint32_t sct[2];  // the dword after each (for the realignment of rows that start off a dword)
  uint32_t bias;
  u32x4 a[ACT_REG ? kActLoads<false, R> : 1];
};
template <bool ACT_REG, int R>
struct Raw<true, ACT_REG, R> {
  u32x4 sc[2];  // columns 4g .. 4g + 3 and 16 + 4g .. 16 + 4g + 3 of the piece
  uint32_t bias;
  u32x4 a[ACT_REG ? kActLoads<true, R> : 1];
};

// Loads every unit issues, whatever else it carries: the two direct weight
// loads (issued last) and the activations from L2.
template <bool FP8, bool ACT_REG, int R>
constexpr int kLoadsPerUnit = 2 + (ACT_REG ? kActLoads<FP8, R> : 0);

// Wait until at most N vector-memory loads of this wave are in flight.  The
// compiler does not track the LDS side of direct loads, so the fences keep
// the LDS reads that follow after the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));  // vmcnt(N) only
  __asm__ volatile("" ::: "memory");
}

// Workgroup barrier for data exchanged through LDS by ds_write / ds_read
// only.  __syncthreads would also wait for every direct load in flight (the
// compiler cannot tell which LDS bytes they write), draining the pipeline.
__device__ __forceinline__ void lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Position of a wave in its flat unit sequence: tile group and unit.
struct Pos {
  int tg, j;
  __device__ __forceinline__ void advance(int nus, int stride) {
    if (++j == nus) {
      j = 0;
      tg += stride;
    }
  }
};

// Activations, two ways (ACT_LDS):
//  * false: loaded from L2 with each unit, at the same pipeline depth;
//  * true: copied once into LDS by the persistent workgroup (rows zero-padded
//    to whole 128-k windows; for FP4 a 256-byte zero block follows the M rows
//    and serves the lanes that carry no row), so the loop issues weight loads
//    only.
// R: FP4 - activation rows per lane (1: M <= 4, four rows per MFMA; 2:
// M <= 8, row pairs); FP8 - result rows a lane scales (1, 2 or 4).  D: units
// in flight ahead of the multiply.
//
// LDS: [kWaves][D + 1] unit slots, [kWaves] scale slices (a wave's slice also
// takes its part of the K-split reduction at the end of a tile), then the
// activation rows (ACT_LDS) or [kWaves] activation staging areas (ACT_REG).
template <typename T, int KS, bool FP8, bool ACT_LDS, int R, int D, bool QDQ>
__global__ __launch_bounds__(64 * kWaves) void gemv_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const void* __restrict__ scales,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int M, int N,
    int K, int cols, FastDiv halves_per_block, FastDiv chunks_per_row, int num_tiles, int nus,
    T* __restrict__ a_work) {
  static_assert(!QDQ || (!FP8 && ACT_LDS), "the W4A4 activation copy is an FP4, LDS-resident mode");
  constexpr bool ACT_REG = !ACT_LDS;
  constexpr int TPW = kWaves / KS;
  constexpr int S = D + 1;          // unit slots (LDS ring and registers)
  constexpr int UW = FP8 ? 1 : 2;   // windows per unit
  constexpr int SU = kScaleUnits<FP8>;
  constexpr int LPU = kLoadsPerUnit<FP8, ACT_REG, R>;
  constexpr uint32_t kSlice = slice_bytes<FP8>();
  typedef Raw<FP8, ACT_REG, R> RawT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;    // fragment side: row li, chunk group g
  const int lr = lane >> 3, lc = lane & 7;    // load side: row lr of an 8-row half, position lc
  const int ks = wave % KS, tw = wave / KS;
  const int NW = (K + 127) >> 7;              // 128-k windows (FP4: the last may hold 32, 64 or 96 k)
  const int NU = (NW + UW - 1) / UW;          // units per row
  const int ntg = (num_tiles + TPW - 1) / TPW;
  const int iters = (ntg - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                    static_cast<int>(gridDim.x);
  // every wave of the workgroup runs the same sequence, so the barriers of
  // the K-split reduction are uniform
  const int total = iters * nus;
  const int stride = gridDim.x;
  const uint32_t row_bytes = FP8 ? static_cast<uint32_t>(K) : static_cast<uint32_t>(K >> 1);
  const uint32_t srow_bytes = FP8 ? static_cast<uint32_t>(cols) * 4u : static_cast<uint32_t>(cols);
  const float ws2 = FP8 ? 1.0f : *ws2p;  // one scalar load, kept in a register

  unsigned char* ring = smem + static_cast<uint32_t>(wave) * (S * kUnitBytes);
  unsigned char* slices = smem + kWaves * S * kUnitBytes;
  unsigned char* slice = slices + wave * kSlice;
  unsigned char* a_lds = slices + kWaves * kSlice;
  const uint32_t lds_pitch = static_cast<uint32_t>(NW) * 256u + 16u;  // bytes per LDS row of A
  const uint32_t zero_off = static_cast<uint32_t>(M) * lds_pitch;       // FP4: the zero block
  const uint32_t a_bytes = static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u;
  const rsrc_t a_rsrc = make_rsrc(A, a_bytes);

  // Per-lane activation offset (bytes, window 0).  FP4, M <= 4: lane
  // (li = 4m' + q, g) carries row m' when q == g; M <= 8: see the row pairs
  // below; a lane that carries no row reads zeros (the zero block in LDS or
  // in the staging area).  FP8: row li (rows >= M are never stored, so
  // lanes li >= M may read any valid row).
  // In the staging area (ACT_REG) the same holds with the staged row pitch.
  uint32_t a_off;
  bool a_valid;
  if constexpr (FP8) {
    a_off = static_cast<uint32_t>(li % M) * (ACT_LDS ? lds_pitch : kStagePitch8);
    a_valid = true;
  } else if constexpr (R == 1) {
    const int m = li >> 2;
    a_valid = (li & 3) == g && m < M;
    a_off = static_cast<uint32_t>(a_valid ? m : 0) * (ACT_LDS ? lds_pitch : kStagePitch4) + 64u * g;
  } else {
    // row pairs: lane (li, g) carries row li >> 1 in the half (li & 1) of
    // the window that its lane group serves (g >> 1), piece g & 1
    const int m = li >> 1;
    a_valid = (li & 1) == (g >> 1) && m < M;
    a_off = static_cast<uint32_t>(a_valid ? m : 0) * (ACT_LDS ? lds_pitch : kStagePitch4) + 128u * (g >> 1) +
            16u * (g & 1);
  }
  // ACT_LDS: the lane's LDS address of window 0 and its step per window; a
  // lane that carries no row keeps reading the zero block (step 0), so the
  // window loop computes each address with one multiply-add
  // (32-bit LDS addresses)
  const lds_cbytes a_win0 = (lds_cbytes)(a_lds + (a_valid ? a_off : zero_off));
  const uint32_t a_wstep = a_valid ? 256u : 0u;
  // ACT_REG: this wave's staging area, the lane's global offset (unit 0) in
  // the row-major loads and its place in the staging area.  FP4 load b:
  // rows 2b + (lane >> 5), 16 bytes at 16 (lane & 31) of the row's 512;
  // FP8 load b: rows 4b + (lane >> 4), 16 bytes at 16 (lane & 15) of 256.
  unsigned char* stage = a_lds + wave * stage_bytes<FP8, R>();
  constexpr int kRowsPerLoad = FP8 ? 4 : 2;
  const int st_row = FP8 ? (lane >> 4) : (lane >> 5);
  const uint32_t st_pos = 16u * static_cast<uint32_t>(FP8 ? (lane & 15) : (lane & 31));
  const uint32_t st_pitch = FP8 ? kStagePitch8 : kStagePitch4;
  const uint32_t unit_act = FP8 ? 256u : 512u;  // activation bytes of a row per unit
  // FP8: scale column of 64-k half window hw (block_size % 64 == 0, so a
  // half lies in one block; halves past the row are clamped to the last)
  auto hcol = [&](int hw) {
    return min(fdiv(static_cast<uint32_t>(min(hw, 2 * NW - 1)), halves_per_block), static_cast<uint32_t>(cols - 1));
  };

  // Window mapping.  Unit u covers bytes 128u .. 128u + 127 of every row.
  // FP4: window 2u + s is bytes 64s .. 64s + 63 of the unit, and lane group g
  // takes chunk 4s + g of it (32 k); FP8: lane group g takes chunks g and
  // 4 + g (k 16g .. + 15 and 64 + 16g .. + 15 of the window).
  // Load side of the pipeline: position and the (wave-uniform) descriptors
  // of its tile, recomputed only when the position enters a new tile.
  Pos lp{static_cast<int>(blockIdx.x), 0};  // next unit to load
  rsrc_t br, sr, biasr;
  auto set_load_tile = [&]() {
    const int t = lp.tg * TPW + tw;
    const int rows = max(0, min(16, N - 16 * t));
    const size_t n0 = static_cast<size_t>(16) * t;
    br = make_rsrc(B + n0 * row_bytes, rows * row_bytes);
    // rounded up to whole dwords: a buffer load checks its range dword by
    // dword, so a row whose last scale bytes share a dword with the end of
    // the array would read them as zero (the bytes past the array in that
    // dword are past the row's last column, and masked)
    sr = make_rsrc(static_cast<const uint8_t*>(scales) + n0 * srow_bytes, (rows * srow_bytes + 3u) & ~3u);
    biasr = make_rsrc(bias + n0, bias ? rows * 2u : 0u);
  };
  set_load_tile();
  // direct-load offsets of the lane (unit 0): row lr (+ 8), chunk lc ^ lr
  // (lr == row & 7).  Rows past the tile's last row are out of range through
  // the descriptor.
  const uint32_t wl = lr * row_bytes + 16u * (lc ^ lr);
  const uint32_t wl8 = wl + 8u * row_bytes;
  // FP4 scale pieces: row lr (+ 8), bytes 16 lc of the 128-byte piece.
  // With K % 64 != 0 a row of K / 16 scale bytes may start off a dword
  // boundary, and buffer loads address whole dwords: the piece is loaded
  // from the dword boundary below, with one dword more, and realigned by
  // sc_shift bytes (the same for rows lr and 8 + lr: 8 * srow_bytes % 4 == 0).
  const uint32_t sl = lr * srow_bytes + 16u * lc;
  const uint32_t sl8 = sl + 8u * srow_bytes;
  const uint32_t sc_shift = sl & 3u;

  auto load = [&](RawT& r, unsigned char* slot) {
    // bias and scale pieces are only requested for the units that carry
    // them (uniform branches; an out-of-range request would still occupy the
    // load pipeline for all 64 lanes)
    if (lp.j == 0) r.bias = buf_load_u16(biasr, 2u * li);
    const int u = ks * nus + lp.j;  // unit of the row
    const bool ok = u < NU;
    const bool piece = ok && lp.j % SU == 0;
    if constexpr (FP8) {
      const int w = u;
      // FP32 scales of columns hcol(2w) .. + 31 (bytes past the row are never used)
      // (the second 16 columns only for 64-k blocks: with larger blocks 16
      // windows span at most 16 columns)
      if (piece) {
        const uint32_t o = li * srow_bytes + 4u * hcol(2 * w) + 16u * g;
        r.sc[0] = buf_load_b128(sr, o);
        if (halves_per_block.d == 1) r.sc[1] = buf_load_b128(sr, o + 64u);
      }
    } else {
      // E4M3 scales of windows 2u .. 2u + 15 (bytes past the row are never used)
      if (piece) {
        r.sc[0] = buf_load_b128(sr, (sl & ~3u) + 16u * u);
        r.sc[1] = buf_load_b128(sr, (sl8 & ~3u) + 16u * u);
        if (srow_bytes & 3u) {  // uniform
          r.sct[0] = buf_load_b32(sr, (sl & ~3u) + 16u * u + 16u);
          r.sct[1] = buf_load_b32(sr, (sl8 & ~3u) + 16u * u + 16u);
        }
      }
    }
    if constexpr (ACT_REG) {
      // row-major activations of the unit's K range; bytes past the end of a
      // row (a last unit with one window) or rows past M read zeros
      const uint32_t kpos = unit_act * static_cast<uint32_t>(u) + st_pos;
#pragma unroll
      for (int b = 0; b < kActLoads<FP8, R>; ++b) {
        const int m = kRowsPerLoad * b + st_row;
        const bool in = m < M && kpos < static_cast<uint32_t>(K) * 2u;
        r.a[b] = buf_load_b128(a_rsrc, in ? static_cast<uint32_t>(m) * static_cast<uint32_t>(K) * 2u + kpos
                                          : kOutOfRange);
      }
    }
    // the unit's weights, last: whatever else is in flight is older
    const uint32_t ub = 128u * static_cast<uint32_t>(u);
    buf_load_lds<16>(br, ok ? wl + ub : kOutOfRange, slot);
    buf_load_lds<16>(br, ok ? wl8 + ub : kOutOfRange, slot + 1024);
    if (++lp.j == nus) {
      lp.j = 0;
      lp.tg += stride;
      set_load_tile();
    }
  };

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t tbias = 0;  // bias bits of the lane's column, current tile
  RawT raw[S];
  Pos cp{static_cast<int>(blockIdx.x), 0};  // unit being multiplied

  if constexpr (ACT_LDS) {
    // Rows 0 .. M-1 of A, zero beyond K, then (FP4) the zero block, by direct
    // loads: LDS chunk q (16 bytes) holds row q / cpr, column q % cpr; the
    // row padding, the zero block and the tail of the last instruction are
    // out-of-range reads, which write zeros and touch no memory.  The fill is
    // requested before the weights, so waiting until only the first D units'
    // weight loads are outstanding means the fill (and the first scale and
    // bias loads) have landed.
    const uint32_t cpr = chunks_per_row.d;  // lds_pitch / 16
    const uint32_t nload = static_cast<uint32_t>(M) * cpr;
    const uint32_t nall = FP8 ? nload : nload + 16u;  // FP4: the 256-byte zero block
    for (uint32_t q0 = 64u * static_cast<uint32_t>(wave); q0 < nall; q0 += 64u * kWaves) {
      const uint32_t q = q0 + static_cast<uint32_t>(lane);
      const uint32_t row = fdiv(q, chunks_per_row), col = q - row * cpr;
      const bool in = q < nload && col * 8u < static_cast<uint32_t>(K);
      buf_load_lds<16>(a_rsrc, in ? row * static_cast<uint32_t>(K) * 2u + col * 16u : kOutOfRange, a_lds + 16u * q0);
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load(raw[d], ring + d * kUnitBytes);
    }
    wait_vm<2 * D>();
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
    if constexpr (QDQ) {
      // W4A4: the copy becomes its NVFP4 quantize-dequantize, in place,
      // block by block (16 k of one row; the row padding and the zero block
      // are zeros and would stay zeros); the first workgroup also writes it
      // to a_work.  The weight loads issued above stay in flight meanwhile.
      typedef typename ActTraits<T>::vec8 V;
      const uint32_t kbr = static_cast<uint32_t>(K) >> 4;  // blocks per row (K % 16 == 0)
      const uint32_t nblk = static_cast<uint32_t>(M) * kbr;
      for (uint32_t b = threadIdx.x; b < nblk; b += 64u * kWaves) {
        const uint32_t m = b / kbr, kb = b - m * kbr;
        unsigned char* p = a_lds + m * lds_pitch + 32u * kb;
        const V x0 = *reinterpret_cast<const V*>(p), x1 = *reinterpret_cast<const V*>(p + 16);
        float v[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[i] = static_cast<float>(x0[i]);
          v[8 + i] = static_cast<float>(x1[i]);
        }
        V r[2];
        nvfp4_qdq_block<T>(v, r);
        *reinterpret_cast<V*>(p) = r[0];
        *reinterpret_cast<V*>(p + 16) = r[1];
        if (blockIdx.x == 0) {
          u32x4* q = reinterpret_cast<u32x4*>(a_work + static_cast<size_t>(m) * K + 16u * kb);
          q[0] = __builtin_bit_cast(u32x4, r[0]);
          q[1] = __builtin_bit_cast(u32x4, r[1]);
        }
      }
      lds_barrier();
    }
  } else {
    // FP4: the staging area's zero block (wave-private: no barrier)
    if constexpr (!FP8)
      if (lane < 8) *reinterpret_cast<u32x4*>(stage + 4u * R * kStagePitch4 + 16u * lane) = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load(raw[d], ring + d * kUnitBytes);
    }
  }

  // multiply one unit (and finish its tile group after the last unit)
  auto consume = [&](const RawT& r, const unsigned char* slot) {
    const int j = cp.j;
    const int u = ks * nus + j;
    if (j == 0) tbias = r.bias;
    typedef ActTraits<T> Tr;
    typedef typename Tr::vec8 V;
    const int sw = li & 7;  // swizzle of the lane's row in the slot
    if constexpr (FP8) {
      // slice rows of kSlicePitch bytes: the 16 rows' scale reads of a
      // window fall in distinct banks
      if (j % SU == 0) {
        *reinterpret_cast<u32x4*>(slice + kSlicePitch * li + 16 * g) = r.sc[0];
        if (halves_per_block.d == 1) *reinterpret_cast<u32x4*>(slice + kSlicePitch * li + 64 + 16 * g) = r.sc[1];
      }
      const int w = min(u, NW - 1);  // windows past NW meet zero weights
      // the scales of this window's two halves, from the piece of the first
      // window of its group (column offsets at most 31)
      const uint32_t c0 = hcol(2 * (ks * nus + (j - j % SU)));
      const uint32_t c_lo = hcol(2 * w), c_hi = hcol(2 * w + 1);
      const float s_lo = *reinterpret_cast<const float*>(slice + kSlicePitch * li + 4 * (c_lo - c0));
      if constexpr (ACT_REG) {
#pragma unroll
        for (int b = 0; b < kActLoads<FP8, R>; ++b)
          *reinterpret_cast<u32x4*>(stage + (kRowsPerLoad * b + st_row) * st_pitch + st_pos) = r.a[b];
      }
      const unsigned char* q = (ACT_LDS ? a_lds + 256u * w : stage) + a_off + 32u * g;
      V a[4];
      a[0] = *reinterpret_cast<const V*>(q);
      a[1] = *reinterpret_cast<const V*>(q + 16u);
      a[2] = *reinterpret_cast<const V*>(q + 128u);
      a[3] = *reinterpret_cast<const V*>(q + 144u);
      wait_vm<D * LPU>();  // this unit's weights have landed
      u32x4 w0 = *reinterpret_cast<const u32x4*>(slot + 128 * li + 16 * (g ^ sw));
      u32x4 w1 = *reinterpret_cast<const u32x4*>(slot + 128 * li + 16 * ((4 + g) ^ sw));
      if ((K & 127) && 128 * (w + 1) > K) {
        // a last window of K % 128 k: the bytes past the row are the next
        // row's E4M3 codes, which may be NaN; zero the lane's chunks past K
        // (K % 16 == 0: whole chunks)
        const u32x4 z = u32x4{0u, 0u, 0u, 0u};
        if (128 * w + 16 * g >= K) w0 = z;
        if (128 * w + 64 + 16 * g >= K) w1 = z;
      }
      // MFMAs 0-1 take k 0 .. 63 of the window, 2-3 k 64 .. 127.  Where
      // both halves lie in one scale block (always, for block_size % 128 ==
      // 0) the four MFMAs make one sum; otherwise each half has its own sum
      // and scale (uniform branch).  The lane holds column n and rows
      // 4g .. 4g + 3.
      f32x4 lo = f32x4{0.f, 0.f, 0.f, 0.f};
      lo = Tr::mfma(a[0], Tr::decode8_fp8(w0.x, w0.y), lo);
      lo = Tr::mfma(a[1], Tr::decode8_fp8(w0.z, w0.w), lo);
      if (c_lo == c_hi) {
        lo = Tr::mfma(a[2], Tr::decode8_fp8(w1.x, w1.y), lo);
        lo = Tr::mfma(a[3], Tr::decode8_fp8(w1.z, w1.w), lo);
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i] = fmaf(lo[i], s_lo, acc[i]);
      } else {
        const float s_hi = *reinterpret_cast<const float*>(slice + kSlicePitch * li + 4 * (c_hi - c0));
        f32x4 hi = f32x4{0.f, 0.f, 0.f, 0.f};
        hi = Tr::mfma(a[2], Tr::decode8_fp8(w1.x, w1.y), hi);
        hi = Tr::mfma(a[3], Tr::decode8_fp8(w1.z, w1.w), hi);
#pragma unroll
        for (int i = 0; i < R; ++i) acc[i] = fmaf(hi[i], s_hi, fmaf(lo[i], s_lo, acc[i]));
      }
    } else {
      if (j % SU == 0) {
        // The piece (scale columns 16u .. 16u + 127 of rows lr and 8 + lr)
        // goes to the slice realigned where rows start off a dword, and with
        // the bytes past the row's last column set to E4M3 zero: they belong
        // to the next row and may hold a NaN code (windows past the row, or a
        // last window of 32, 64 or 96 k).  Both steps are skipped where they
        // change nothing (uniform branches).
        u32x4 v0 = r.sc[0], v1 = r.sc[1];
        if (srow_bytes & 3u) {
          auto realign = [&](const u32x4& v, uint32_t t) {
            return u32x4{__builtin_amdgcn_alignbyte(v.y, v.x, sc_shift), __builtin_amdgcn_alignbyte(v.z, v.y, sc_shift),
                         __builtin_amdgcn_alignbyte(v.w, v.z, sc_shift), __builtin_amdgcn_alignbyte(t, v.w, sc_shift)};
          };
          v0 = realign(v0, r.sct[0]);
          v1 = realign(v1, r.sct[1]);
        }
        if (16 * u + 128 > cols) {
          const int vb = cols - 16 * u - 16 * lc;  // valid bytes of the lane's 16
          u32x4 m;
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const int nv = vb - 4 * d;
            m[d] = nv >= 4 ? ~0u : nv <= 0 ? 0u : (1u << (8 * nv)) - 1u;
          }
          v0 &= m;
          v1 &= m;
        }
        *reinterpret_cast<u32x4*>(slice + kSlicePitch * lr + 16 * lc) = v0;
        *reinterpret_cast<u32x4*>(slice + kSlicePitch * (8 + lr) + 16 * lc) = v1;
      }
      if constexpr (ACT_REG) {
#pragma unroll
        for (int b = 0; b < kActLoads<FP8, R>; ++b)
          *reinterpret_cast<u32x4*>(stage + (kRowsPerLoad * b + st_row) * st_pitch + st_pos) = r.a[b];
      }
      wait_vm<D * LPU>();  // this unit's weights have landed
      // Every LDS read of the unit's two windows is issued before either
      // window's arithmetic, so that the second window's reads overlap the
      // first window's work.
      u32x2 sb[2];
      u32x4 av[2][4];
      u32x4 wv[2];
      // activation fragment i of a window: 16 bytes at 16 i (M <= 4) or 32 i
      // (row pairs) from the lane's offset
      constexpr uint32_t kAStep = R == 1 ? 16u : 32u;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int wa = min(2 * u + s2, NW - 1);  // windows past NW meet zero scales (zeroed in the slice)
        sb[s2] = *reinterpret_cast<const u32x2*>(slice + kSlicePitch * li + 8 * (2 * (j % SU) + s2));
        if constexpr (ACT_LDS) {
          const lds_cbytes q = a_win0 + __umul24(a_wstep, static_cast<uint32_t>(wa));
#pragma unroll
          for (int i = 0; i < 4; ++i) av[s2][i] = *reinterpret_cast<const lds_u32x4*>(q + kAStep * i);
        } else {
          const unsigned char* q = stage + (a_valid ? a_off + 256u * s2 : 4u * R * kStagePitch4);
#pragma unroll
          for (int i = 0; i < 4; ++i) av[s2][i] = *reinterpret_cast<const u32x4*>(q + kAStep * i);
        }
        if constexpr (R == 1) {
          // chunk 4 s2 + g of row li (32 codes, blocks 2g and 2g + 1 of the
          // window); dword 2s + p holds piece p of block 2g + s
          wv[s2] = *reinterpret_cast<const u32x4*>(slot + 128 * li + 16 * ((4 * s2 + g) ^ sw));
        } else {
          // row pairs: dword t is piece g & 1 of block 4 (g >> 1) + t, from
          // chunks 4 s2 + 2 (g >> 1) (t = 0, 1) and the next (t = 2, 3)
          const int c = 4 * s2 + 2 * (g >> 1);
          const unsigned char* p0 = slot + 128 * li + 16 * (c ^ sw) + 4 * (g & 1);
          const unsigned char* p1 = slot + 128 * li + 16 * ((c + 1) ^ sw) + 4 * (g & 1);
          wv[s2] = u32x4{*reinterpret_cast<const uint32_t*>(p0), *reinterpret_cast<const uint32_t*>(p0 + 8),
                         *reinterpret_cast<const uint32_t*>(p1), *reinterpret_cast<const uint32_t*>(p1 + 8)};
        }
      }
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        V bw[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) bw[i] = Tr::decode8_fp4(wv[s2][i]);
        const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
        // scale of block b of the window: byte b
        auto scales = [&](float (&sc)[8]) {
          const f32x2 s01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(sb[s2].x), false);
          const f32x2 s23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(sb[s2].x), true);
          const f32x2 s45 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(sb[s2].y), false);
          const f32x2 s67 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(sb[s2].y), true);
          sc[0] = s01.x; sc[1] = s01.y; sc[2] = s23.x; sc[3] = s23.y;
          sc[4] = s45.x; sc[5] = s45.y; sc[6] = s67.x; sc[7] = s67.y;
        };
        float sc[8];
        if constexpr (R == 1) {
          f32x4 d[2];
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            d[s] = Tr::mfma(__builtin_bit_cast(V, av[s2][2 * s]), bw[2 * s], zero);
            d[s] = Tr::mfma(__builtin_bit_cast(V, av[s2][2 * s + 1]), bw[2 * s + 1], d[s]);
          }
          scales(sc);
          // result row rr of set s is block 2 rr + s of row g
#pragma unroll
          for (int rr = 0; rr < 4; ++rr)
#pragma unroll
            for (int s = 0; s < 2; ++s) acc[0] = fmaf(d[s][rr], sc[2 * rr + s], acc[0]);
        } else {
          // MFMA t: result row r is block 4 (r & 1) + t of row 2g + (r >> 1)
          scales(sc);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const f32x4 d = Tr::mfma(__builtin_bit_cast(V, av[s2][t]), bw[t], zero);
            acc[0] = fmaf(d[0], sc[t], acc[0]);
            acc[0] = fmaf(d[1], sc[4 + t], acc[0]);
            acc[1] = fmaf(d[2], sc[t], acc[1]);
            acc[1] = fmaf(d[3], sc[4 + t], acc[1]);
          }
        }
      }
    }
    if (j == nus - 1) {
      // end of this tile group: reduce the K split through the slices (every
      // wave has read its scales for this unit), then the epilogue (uniform
      // across the workgroup: every wave has the same sequence)
      if (KS > 1) {
        *reinterpret_cast<f32x4*>(slice + 16 * lane) = acc;
        lds_barrier();
        if (ks == 0) {
#pragma unroll
          for (int v = 1; v < KS; ++v) acc += *reinterpret_cast<const f32x4*>(slices + (wave + v) * kSlice + 16 * lane);
        }
        lds_barrier();
      }
      if (ks == 0) {
        const int n = 16 * (cp.tg * TPW + tw) + li;
        if (n < N) {
          // zero bits when there is no bias (zero-length buffer)
          const float b = static_cast<float>(__builtin_bit_cast(T, static_cast<uint16_t>(tbias)));
          if constexpr (FP8) {
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const int m = 4 * g + r4;
              if (m < M) Y[static_cast<size_t>(m) * N + n] = round_to<T>(acc[r4] + b);
            }
          } else {
#pragma unroll
            for (int h = 0; h < R; ++h) {
              const int m = R == 1 ? g : 2 * g + h;  // the lane's rows
              if (m < M) Y[static_cast<size_t>(m) * N + n] = round_to<T>(fmaf(acc[h], ws2, b));
            }
          }
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    cp.advance(nus, stride);
  };

  // Unit f sits in slot f % S.  Loads run ahead unconditionally (past the end
  // they are out of range), so every step waits only for its own, oldest,
  // loads; steps past the end of the sequence skip the multiply (the
  // condition is uniform across the workgroup).
  for (int f0 = 0; f0 < total; f0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      load(raw[(u + D) % S], ring + ((u + D) % S) * kUnitBytes);
      if (f0 + u < total) consume(raw[u], ring + u * kUnitBytes);
    }
  }
}

// --------------------------------------------------------------------- launch

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// Kernel variants by where the activations live and the pipeline depth
// (units in flight per wave): MODE 0 - streamed from L2 with each unit, 4
// units; 1 - in LDS, 2 units; 2 - in LDS, 4 units (the deepest ring that
// leaves room for them).
template <bool FP8, int MODE, int R>
constexpr int depth() {
  return MODE == 1 ? 2 : 4;
}

size_t lds_bytes(int mode, bool fp8, int M, int NW) {
  const size_t ring = kWaves * (static_cast<size_t>(mode == 1 ? 2 : 4) + 1) * kUnitBytes;
  const size_t slices = kWaves * static_cast<size_t>(fp8 ? slice_bytes<true>() : slice_bytes<false>());
  // ACT_LDS: the M rows (FP4: plus the 256-byte zero block); ACT_REG: the
  // staging areas
  const size_t stage = fp8 ? stage_bytes<true, 1>() : M > 4 ? stage_bytes<false, 2>() : stage_bytes<false, 1>();
  // ACT_LDS: whole direct-load instructions of 64 chunks of 16 bytes
  const size_t act_chunks = static_cast<size_t>(M) * (static_cast<size_t>(NW) * 16 + 1) + (fp8 ? 0 : 16);
  const size_t act = mode > 0 ? (act_chunks + 63) / 64 * 1024 : kWaves * stage;
  return ring + slices + act;
}

template <typename T, int KS, bool FP8, int MODE, int R, bool QDQ = false>
constexpr auto kernel_ptr() {
  return &gemv_kernel<T, KS, FP8, (MODE > 0), R, depth<FP8, MODE, R>(), QDQ>;
}

// Dynamic LDS above 64 KiB must be allowed per kernel, once per device.
template <typename T, int KS, bool FP8, int MODE, int R, bool QDQ = false>
void allow_lds() {
  static std::once_flag once[kMaxDevices];
  once_per_device(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel_ptr<T, KS, FP8, MODE, R, QDQ>()),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kMaxLds));
  });
}

// Resident workgroups per CU for a kernel variant and LDS size.
template <typename T, int KS, bool FP8, int MODE, int R>
int wg_per_cu(size_t lds) {
  allow_lds<T, KS, FP8, MODE, R>();
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel_ptr<T, KS, FP8, MODE, R>(), 64 * kWaves, lds) !=
          hipSuccess ||
      v < 1)
    v = 1;
  return v;
}

template <typename T, int KS, bool FP8, int MODE>
int wg_per_cu_r(int R, size_t lds) {
  if (R == 1) return wg_per_cu<T, KS, FP8, MODE, 1>(lds);
  if (R == 2 || !FP8) return wg_per_cu<T, KS, FP8, MODE, 2>(lds);
  return wg_per_cu<T, KS, FP8, MODE, (FP8 ? 4 : 2)>(lds);
}

template <typename T, bool FP8, int MODE>
int slots_for(int KS, int R, int M, int NW) {
  const size_t lds = lds_bytes(MODE, FP8, M, NW);
  int per = 1;
  switch (KS) {
    case 1: per = wg_per_cu_r<T, 1, FP8, MODE>(R, lds); break;
    case 2: per = wg_per_cu_r<T, 2, FP8, MODE>(R, lds); break;
    case 4: per = wg_per_cu_r<T, 4, FP8, MODE>(R, lds); break;
    default: per = wg_per_cu_r<T, 8, FP8, MODE>(R, lds); break;
  }
  return device_cus() * per;
}

struct Plan {
  int KS, grid, nus, mode;
};

// Launch plan.  Activations go to LDS whenever they fit (reading them from
// L2 per window costs more load instructions than the weights themselves),
// with the deep ring when it fits beside them.  The K split KS (and with it
// TPW = 8 / KS tiles side by side) is the one with the least work on the
// busiest wave: rounds of tile groups per workgroup (persistent workgroups,
// at most the resident ones) times units per wave, counting the units a wave
// pads with when KS does not divide the row.  Ties go to the split with fewer padded units, then to the larger
// split; every wave keeps at least one unit.
template <typename T, bool FP8>
int slots_mode(int mode, int ks, int R, int M, int NW) {
  return mode == 2 ? slots_for<T, FP8, 2>(ks, R, M, NW)
                   : mode == 1 ? slots_for<T, FP8, 1>(ks, R, M, NW) : slots_for<T, FP8, 0>(ks, R, M, NW);
}

template <typename T, bool FP8>
Plan plan(int64_t N, int M, int R, int NW) {
  const int64_t tiles = (N + 15) / 16;
  const int NU = FP8 ? NW : (NW + 1) / 2;
  const int mode = lds_bytes(2, FP8, M, NW) <= kMaxLds ? 2 : lds_bytes(1, FP8, M, NW) <= kMaxLds ? 1 : 0;
  Plan best{1, 1, NU, mode};
  int64_t best_cost = -1;
  int best_pad = 0;
  for (int ks = 8; ks >= 1; ks >>= 1) {
    if (NU < ks) continue;
    const int64_t ntg = (tiles + kWaves / ks - 1) / (kWaves / ks);
    const int64_t slots = slots_mode<T, FP8>(mode, ks, R, M, NW);
    // rounds of tile groups on the resident workgroups, then as few
    // workgroups as give every one the same number of rounds (one less for
    // some): a last, partial round would run on few CUs, each held to its own
    // memory rate, while the same bytes spread over all rounds keep HBM busy
    const int64_t rounds = (ntg + slots - 1) / slots;
    const int64_t grid = (ntg + rounds - 1) / rounds;
    const int nus = (NU + ks - 1) / ks;
    const int64_t cost = rounds * nus;
    const int pad = nus * ks - NU;
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && pad < best_pad)) {
      best_cost = cost;
      best_pad = pad;
      best = Plan{ks, static_cast<int>(grid), nus, mode};
    }
  }
  return best;
}

// The plan depends only on the sizes, the device and the variant's resource
// use; it is computed once per shape (the occupancy queries cost several
// microseconds, more than a decode GEMV takes on the GPU).
struct PlanEntry {
  int64_t N;
  int M, NW, dev, kind;
  Plan p;
};

template <typename T, bool FP8>
Plan cached_plan(int64_t N, int M, int R, int NW) {
  constexpr int kEntries = 64;
  static PlanEntry table[kEntries];
  static int used = 0, next = 0;
  static std::mutex mu;
  const int kind = (FP8 ? 2 : 0) + (sizeof(T) == 2 && __is_same(T, __bf16) ? 1 : 0);
  int dev = 0;
  (void)hipGetDevice(&dev);
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i) {
      const PlanEntry& e = table[i];
      if (e.N == N && e.M == M && e.NW == NW && e.dev == dev && e.kind == kind) return e.p;
    }
  }
  const Plan p = plan<T, FP8>(N, M, R, NW);
  std::lock_guard<std::mutex> lock(mu);
  table[next] = PlanEntry{N, M, NW, dev, kind, p};
  next = (next + 1) % kEntries;
  if (used < kEntries) ++used;
  return p;
}

template <typename T, int KS, bool FP8, int MODE, bool QDQ>
void launch_v(const MatmulArgs& a, const Plan& p, int R, size_t lds, FastDiv wpb, FastDiv cpr, int tiles,
              T* a_work) {
  hipStream_t s = static_cast<hipStream_t>(a.stream);
#define FP4W_GEMV_LAUNCH(R_)                                                                            \
  allow_lds<T, KS, FP8, MODE, R_, QDQ>();                                                               \
  hipLaunchKernelGGL((kernel_ptr<T, KS, FP8, MODE, R_, QDQ>()), dim3(p.grid), dim3(64 * kWaves), lds,   \
                     s, static_cast<const T*>(a.A), a.B, a.scales, a.ws2, static_cast<const T*>(a.bias), \
                     static_cast<T*>(a.Y), static_cast<int>(a.M), static_cast<int>(a.N),                \
                     static_cast<int>(a.K), static_cast<int>(a.scale_cols), wpb, cpr, tiles, p.nus,     \
                     a_work)
  if (R == 1) {
    FP4W_GEMV_LAUNCH(1);
  } else if (R == 2) {
    FP4W_GEMV_LAUNCH(2);
  } else if constexpr (FP8) {
    FP4W_GEMV_LAUNCH(4);
  }
#undef FP4W_GEMV_LAUNCH
}

template <typename T, bool FP8, int MODE, bool QDQ>
void launch_mode(const MatmulArgs& a, const Plan& p, int R, size_t lds, FastDiv wpb, FastDiv cpr, int tiles,
                 T* a_work) {
  switch (p.KS) {
    case 1: launch_v<T, 1, FP8, MODE, QDQ>(a, p, R, lds, wpb, cpr, tiles, a_work); break;
    case 2: launch_v<T, 2, FP8, MODE, QDQ>(a, p, R, lds, wpb, cpr, tiles, a_work); break;
    case 4: launch_v<T, 4, FP8, MODE, QDQ>(a, p, R, lds, wpb, cpr, tiles, a_work); break;
    default: launch_v<T, 8, FP8, MODE, QDQ>(a, p, R, lds, wpb, cpr, tiles, a_work); break;
  }
}

// QDQ (W4A4, FP4 only): the activation copy in LDS is quantize-dequantized
// in place and written to a_work; returns 1, launching nothing, when the
// activations do not fit in LDS (the copy is not made).
template <typename T, bool FP8, bool QDQ = false>
int launch_t(const MatmulArgs& a, T* a_work = nullptr) {
  // buffer offsets are 32-bit: one 16-column tile and the activations must fit
  if (a.N > 0x7fffffff - 16 || a.K > (int64_t(1) << 26) || a.M * a.K * 2 >= (int64_t(1) << 31))
    return -1;
  const int M = static_cast<int>(a.M);
  const int NW = static_cast<int>((a.K + 127) / 128);
  // FP8: result rows a lane scales; FP4: activation rows per lane
  const int R = FP8 ? (M >= 3 ? 4 : M) : (M > 4 ? 2 : 1);
  const Plan p = cached_plan<T, FP8>(a.N, M, R, NW);
  const int tiles = static_cast<int>((a.N + 15) / 16);
  const size_t lds = lds_bytes(p.mode, FP8, M, NW);
  const FastDiv wpb = make_fastdiv(FP8 ? static_cast<uint32_t>(a.block_size / 64) : 1u);  // FP8: halves per block
  const FastDiv cpr = make_fastdiv(static_cast<uint32_t>(NW) * 16u + 1u);  // 16-byte chunks per LDS row
  if constexpr (QDQ) {
    // Every workgroup quantizes the whole of A again, so the fused form pays
    // off only for small M x K: up to 3 blocks of 16 per thread it beat the
    // separate QDQ launch (M = 4, K = 5120: 8.7 against 9.4 us), at 5 it lost
    // (M = 8: about 11 against 10.1 us).
    if (p.mode == 0 || a.M * (a.K / 16) > 3 * 64 * kWaves) return 1;
  }
  if (p.mode == 2)
    launch_mode<T, FP8, 2, QDQ>(a, p, R, lds, wpb, cpr, tiles, a_work);
  else if (p.mode == 1)
    launch_mode<T, FP8, 1, QDQ>(a, p, R, lds, wpb, cpr, tiles, a_work);
  else if constexpr (!QDQ)
    launch_mode<T, FP8, 0, false>(a, p, R, lds, wpb, cpr, tiles, a_work);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_fp4_gemv(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_t<__bf16, false>(a) : launch_t<_Float16, false>(a);
}

int launch_fp4_gemv_w4a4(const MatmulArgs& a, void* a_work) {
  return a.act == Act::BF16 ? launch_t<__bf16, false, true>(a, static_cast<__bf16*>(a_work))
                            : launch_t<_Float16, false, true>(a, static_cast<_Float16*>(a_work));
}

int launch_fp8_gemv(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_t<__bf16, true>(a) : launch_t<_Float16, true>(a);
}

}  // namespace fp4w

// Skinny matmul (M <= 64: batched decode, short prefill chunks) for
// weight-only FP4 and FP8, on MFMA.
//
// Still memory-bound on the weights: at M <= 64 a weight byte feeds at most
// 256 FLOP, below the FLOP/byte balance of the chip, so the kernel is built
// like the decode GEMV: every packed weight byte is streamed from HBM once
// with 16-byte loads, a wave owns 16 output columns, the KS waves of a
// workgroup split K, and a persistent workgroup runs one flat pipeline over
// all its tiles.  The big-tile GEMM would give such shapes only N / 256
// workgroups.
//
// What differs from the GEMV is the MFMA layout.  The activation rows fill
// the A operand directly (row tile t holds rows 16 t .. 16 t + 15; rows past
// M read zeros), so a 128-k window costs 4 MFMAs per row tile, against four
// per four rows for the GEMV's block-diagonal scheme.  The block scale
// therefore has to be inside the B operand:
//  * FP4: E2M1 x E4M3 is exact in FP16 and BF16 ([FP4 doc] §4, tensor-core
//    sub-path, exactness argument), so each 16-k block is decoded already
//    scaled; weight_scale_2 and the bias are applied in the epilogue.
//  * FP8: E4M3 -> T is exact; block_size % 128 == 0 puts a whole window in
//    one scale block, so the window is accumulated in a fresh MFMA
//    accumulator and added with its FP32 scale ([FP8 doc] §2), as the GEMV
//    does.
// The decode cost is shared by all row tiles.
//
// K mapping (a reduction axis: both operands only have to agree).  Window w
// covers k = 128 w .. 128 w + 127; in MFMA step i lane group g supplies the
// 8-k unit 4 g + i of it (k 128 w + 32 g + 8 i .. + 7), for the weights and
// the activations alike, so a lane's four steps take one contiguous 32-k
// chunk of its column: one 16-byte fragment (FP4) or two (FP8).
//  * FP4 steps 0, 1 lie in block 8 w + 2 g, steps 2, 3 in block 8 w + 2 g + 1.
//  * Weights travel global -> LDS by direct loads: a unit is 128 contiguous
//    bytes of each of the wave's 16 rows (two FP4 windows, one FP8 window),
//    fetched by two instructions of 8 rows x 128 bytes.  HBM streams at full
//    rate only for whole 128-byte lines per instruction; 16 rows x 64 bytes
//    (the register-direct MFMA layout) reaches about two thirds of it.  Each
//    row's chunks are loaded in the order chunk ^ (row & 7), so the fragment
//    reads are free of bank conflicts.  A wave has a private ring and waits
//    for its own loads only.
//  * FP4 scale bytes travel in 128-byte pieces per row (16 windows), parked in
//    a per-wave LDS slice.
//
// Activations come from L2 (at most M x K x 2 bytes, read by every
// workgroup) in the same pipeline slot as the weights: loads retire in
// order, so a shallower activation stream would also drain the weight
// stream.  That costs registers: the depth falls as the row tiles grow.
// Their cost is set by how many rows one load instruction touches, not by
// the bytes: a load in the MFMA layout touches 16 rows; loaded row-major
// instead (4 rows x 256 contiguous bytes per instruction) the same bytes
// cost about half the time.  So a window's activations are loaded
// row-major and moved into the MFMA layout through a wave-private LDS
// staging area, one row tile at a time (16-byte chunks XOR-swizzled by row,
// conflict-free on both the write and the read side), which also holds the
// K-split reduction at the end of a tile.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"

#include <hip/hip_runtime.h>

#include <mutex>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr int kSkWaves = 8;  // waves per workgroup (KS x TPW)

// One window of one lane, in registers: the block scales (FP4: the piece of
// 16 windows, first window of each piece; FP8: the window's FP32 scale), the
// bias bits (first window of a tile) and 4 x 16 activation bytes per row
// tile (row-major: load q of tile t holds rows 16 t + 4 q .. + 3).  The
// weights go to LDS by direct loads.
template <bool FP8, int MT>
struct SkRaw;
template <int MT>
struct SkRaw<false, MT> {
  u32x4 sc[2];  // scale rows lr and 8 + lr, 16 bytes each
  uint32_t bias;
  u32x4 a[4 * MT];
};
template <int MT>
struct SkRaw<true, MT> {
  uint32_t sc;  // FP32 block scale bits
  uint32_t bias;
  u32x4 a[4 * MT];
};

constexpr uint32_t kSkUnit = 2048;      // weight slot: 16 rows x 128 bytes
constexpr uint32_t kSkScratch = 4096;   // activation staging: 16 rows x 256 bytes
constexpr int kSkSlicePitch = 144;      // FP4 scale slice: bytes per row (128 + 16)
constexpr uint32_t kSkSlice = 16 * kSkSlicePitch;

// Weight slots of a wave's ring.  A unit is 128 contiguous bytes of each of
// the wave's 16 rows: two windows for FP4 (loaded every second step), one
// for FP8.  A slot is refilled only after the last step that reads it.
template <bool FP8, int D>
constexpr int sk_ring() {
  return FP8 ? D + 1 : (D + 1) / 2 + 1;
}

template <bool FP8, int D>
constexpr uint32_t sk_lds_per_wave() {
  return static_cast<uint32_t>(sk_ring<FP8, D>()) * kSkUnit + kSkScratch + (FP8 ? 0u : kSkSlice);
}

// Wait until at most N vector-memory loads of this wave are in flight.  The
// compiler does not track the LDS side of direct loads, so the fences keep
// the LDS reads that follow after the wait.
template <int N>
__device__ __forceinline__ void sk_wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));  // vmcnt(N) only
  __asm__ volatile("" ::: "memory");
}

// Workgroup barrier for data exchanged through LDS by ds_write / ds_read only
// (__syncthreads would also wait for the direct loads in flight).
__device__ __forceinline__ void sk_lds_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

struct SkPos {
  int tg, j;
  __device__ __forceinline__ void advance(int nws, int stride) {
    if (++j == nws) {
      j = 0;
      tg += stride;
    }
  }
};

template <typename T, bool FP8, int MT, int KS, int D>
__global__ __launch_bounds__(64 * kSkWaves) void skinny_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const void* __restrict__ scales,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int M, int N, int K,
    int cols, FastDiv win_per_block, int num_tiles, int nws) {
  constexpr int TPW = kSkWaves / KS;
  constexpr int S = D + 1;
  constexpr int NS = sk_ring<FP8, D>();
  constexpr uint32_t kWaveLds = sk_lds_per_wave<FP8, D>();
  typedef SkRaw<FP8, MT> RawT;
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  // per wave: the weight ring, the activation staging area (also the K-split
  // partial sums at the end of a tile) and (FP4) the scale slice
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int lr = lane >> 3, lc = lane & 7;  // direct loads: row lr of an 8-row half, position lc
  const int ks = wave % KS, tw = wave / KS;
  unsigned char* ring = smem + wave * kWaveLds;
  unsigned char* scr = ring + NS * kSkUnit;
  unsigned char* slice = scr + kSkScratch;
  const int NW = K >> 7;
  const int ntg = (num_tiles + TPW - 1) / TPW;
  const int iters = (ntg - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                    static_cast<int>(gridDim.x);
  const int total = iters * nws;  // the same on every wave: reduction barriers are uniform
  const int stride = gridDim.x;
  const uint32_t row_bytes = FP8 ? static_cast<uint32_t>(K) : static_cast<uint32_t>(K >> 1);
  const uint32_t srow_bytes = FP8 ? static_cast<uint32_t>(cols) * 4u : static_cast<uint32_t>(cols);
  const float ws2 = FP8 ? 1.0f : *ws2p;
  const rsrc_t a_rsrc = make_rsrc(A, static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u);

  // row-major activation loads: lane l reads 16 bytes (chunk l % 16 of the
  // window) of row 16 t + 4 q + l / 16; rows past M read zeros
  const uint32_t row_pitch = static_cast<uint32_t>(K) * 2u;
  const uint32_t a_lane = static_cast<uint32_t>(g) * row_pitch + 16u * static_cast<uint32_t>(li);
  // LDS byte offsets of the staging area: the chunk this lane writes (load q
  // adds 1024 q and XORs the chunk with 4 q: chunk c of row r sits at
  // position c ^ r), and the chunk it reads for MFMA step i: row li, chunk
  // 4 g + i, i.e. r_lds ^ 16 i
  const uint32_t w_lds = static_cast<uint32_t>(g) * 256u + 16u * static_cast<uint32_t>(li ^ g);
  const uint32_t r_lds = static_cast<uint32_t>(li) * 256u + 16u * static_cast<uint32_t>((4 * g) ^ li);
  // Weights: direct loads of row lr (+ 8), chunk lc ^ lr (lr == row & 7), so
  // chunk c of row r sits at position c ^ (r & 7) of its 128-byte row.  The
  // lane's fragment: FP4 window s of the unit, chunk 4 s + g (dword i = 8-k
  // unit 4 g + i of the window, MFMA step i); FP8 chunks 2 g and 2 g + 1
  // (step i: chunk 2 g + i / 2, dwords 2 (i & 1) and 2 (i & 1) + 1).
  const int sw = li & 7;
  const uint32_t wf0 = 128u * li + 16u * static_cast<uint32_t>(FP8 ? ((2 * g) ^ sw) : (g ^ sw));
  const uint32_t wf1 = 128u * li + 16u * static_cast<uint32_t>(FP8 ? ((2 * g + 1) ^ sw) : ((4 + g) ^ sw));
  const uint32_t wl = lr * row_bytes + 16u * static_cast<uint32_t>(lc ^ lr);
  const uint32_t wl8 = wl + 8u * row_bytes;
  // FP4 scale pieces (16 windows = 128 bytes of a row): rows lr (+ 8), bytes
  // 16 lc of the piece
  const uint32_t sl = lr * srow_bytes + 16u * lc;
  const uint32_t sl8 = sl + 8u * srow_bytes;
  auto scol = [&](int w) {  // FP8 scale column of window w
    return min(fdiv(static_cast<uint32_t>(w), win_per_block), static_cast<uint32_t>(cols - 1));
  };

  SkPos lp{static_cast<int>(blockIdx.x), 0};
  rsrc_t br, sr, biasr;
  auto set_load_tile = [&]() {
    const int t = lp.tg * TPW + tw;
    const int rows = max(0, min(16, N - 16 * t));  // 0 past the last tile: every load reads zeros
    const size_t n0 = static_cast<size_t>(16) * t;
    br = make_rsrc(B + n0 * row_bytes, rows * row_bytes);
    sr = make_rsrc(static_cast<const uint8_t*>(scales) + n0 * srow_bytes, rows * srow_bytes);
    biasr = make_rsrc(bias + n0, bias ? rows * 2u : 0u);
  };
  set_load_tile();

  int lslot = 0;  // ring slot of the next unit to load
  auto load = [&](RawT& r) {
    if (lp.j == 0) r.bias = buf_load_u16(biasr, 2u * li);
    const int w = ks * nws + lp.j;
    const bool ok = w < NW;  // windows past K read zeros (weights, scales, activations)
    if constexpr (FP8) {
      r.sc = buf_load_b32(sr, ok ? li * srow_bytes + 4u * scol(w) : kOutOfRange);
    } else {
      if (lp.j % 16 == 0) {  // E4M3 scales of windows w .. w + 15 (bytes past the row are never used)
        r.sc[0] = buf_load_b128(sr, ok ? sl + 8u * w : kOutOfRange);
        r.sc[1] = buf_load_b128(sr, ok ? sl8 + 8u * w : kOutOfRange);
      }
    }
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r0 = 16 * t + 4 * q;  // first row of this load
        const bool valid = ok && g < M - r0;
        r.a[4 * t + q] = buf_load_b128(
            a_rsrc, valid ? a_lane + static_cast<uint32_t>(r0) * row_pitch + 256u * w : kOutOfRange);
      }
    // the unit's weights, last (FP4: at the first window of the unit)
    if (FP8 || (lp.j & 1) == 0) {
      const uint32_t ub = (FP8 ? 128u : 64u) * static_cast<uint32_t>(w);
      unsigned char* dst = ring + lslot * kSkUnit;
      buf_load_lds<16>(br, ok ? wl + ub : kOutOfRange, dst);
      buf_load_lds<16>(br, ok ? wl8 + ub : kOutOfRange, dst + 1024);
      lslot = lslot + 1 == NS ? 0 : lslot + 1;
    }
    if (++lp.j == nws) {
      lp.j = 0;
      lp.tg += stride;
      set_load_tile();
    }
  };

  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t tbias = 0;
  RawT raw[S];
  SkPos cp{static_cast<int>(blockIdx.x), 0};
  int cslot = 0;  // ring slot of the unit being multiplied

#pragma unroll
  for (int d = 0; d < D; ++d) load(raw[d]);

  auto consume = [&](const RawT& r) {
    const int j = cp.j;
    const int w = ks * nws + j;
    if (j == 0) tbias = r.bias;
    V bw[4];
    float scf = 1.0f;
    if constexpr (FP8) {
      sk_wait_vm<D*(4 * MT + 3)>();  // this window's weights have landed
      const unsigned char* slot = ring + cslot * kSkUnit;
      const u32x4 c0 = *reinterpret_cast<const u32x4*>(slot + wf0);
      const u32x4 c1 = *reinterpret_cast<const u32x4*>(slot + wf1);
      bw[0] = Tr::decode8_fp8(c0.x, c0.y);
      bw[1] = Tr::decode8_fp8(c0.z, c0.w);
      bw[2] = Tr::decode8_fp8(c1.x, c1.y);
      bw[3] = Tr::decode8_fp8(c1.z, c1.w);
      scf = __builtin_bit_cast(float, r.sc);
      cslot = cslot + 1 == NS ? 0 : cslot + 1;
    } else {
      if (j % 16 == 0) {
        *reinterpret_cast<u32x4*>(slice + kSkSlicePitch * lr + 16 * lc) = r.sc[0];
        *reinterpret_cast<u32x4*>(slice + kSkSlicePitch * (8 + lr) + 16 * lc) = r.sc[1];
      }
      if ((j & 1) == 0) sk_wait_vm<D * 4 * MT>();  // this unit's weights have landed
      const unsigned char* slot = ring + cslot * kSkUnit;
      const u32x4 wv = *reinterpret_cast<const u32x4*>(slot + ((j & 1) ? wf1 : wf0));
      // scales of blocks 2 g (steps 0, 1) and 2 g + 1 (steps 2, 3) of the
      // window, folded into the operand (exact); windows past K get zero
      const uint32_t sb =
          w < NW ? *reinterpret_cast<const uint16_t*>(slice + kSkSlicePitch * li + 8 * (j % 16) + 2 * g) : 0u;
      const float s0 = e4m3_to_f32<0>(sb), s1 = e4m3_to_f32<1>(sb);
      bw[0] = Tr::decode8(wv.x, Tr::make_scale(s0));
      bw[1] = Tr::decode8(wv.y, Tr::make_scale(s0));
      bw[2] = Tr::decode8(wv.z, Tr::make_scale(s1));
      bw[3] = Tr::decode8(wv.w, Tr::make_scale(s1));
      if (j & 1) cslot = cslot + 1 == NS ? 0 : cslot + 1;
    }
    // activations, one row tile at a time: row-major chunks into the staging
    // area, back in the MFMA layout (same wave, so LDS order needs no wait)
#pragma unroll
    for (int t = 0; t < MT; ++t) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(scr + 1024 * q + (w_lds ^ (64u * q))) = r.a[4 * t + q];
      V av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = *reinterpret_cast<const V*>(scr + (r_lds ^ (16u * i)));
      if constexpr (FP8) {
        f32x4 blk = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) blk = Tr::mfma(av[i], bw[i], blk);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = fmaf(blk[q], scf, acc[t][q]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t] = Tr::mfma(av[i], bw[i], acc[t]);
      }
    }
    if (j == nws - 1) {
      // end of a tile: reduce the K split through the staging areas (this
      // wave's reads of them were issued before these writes), then the
      // epilogue
      if (KS > 1) {
#pragma unroll
        for (int t = 0; t < MT; ++t) *reinterpret_cast<f32x4*>(scr + 1024 * t + 16 * lane) = acc[t];
        sk_lds_barrier();
        if (ks == 0) {
#pragma unroll
          for (int v = 1; v < KS; ++v)
#pragma unroll
            for (int t = 0; t < MT; ++t)
              acc[t] += *reinterpret_cast<const f32x4*>(smem + (wave + v) * kWaveLds + NS * kSkUnit + 1024 * t +
                                                        16 * lane);
        }
        sk_lds_barrier();
      }
      if (ks == 0) {
        const int n = 16 * (cp.tg * TPW + tw) + li;
        if (n < N) {
          const float b = static_cast<float>(__builtin_bit_cast(T, static_cast<uint16_t>(tbias)));
          // result lane (column li, group g) holds rows 16 t + 4 g .. + 3
#pragma unroll
          for (int t = 0; t < MT; ++t)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int m = 16 * t + 4 * g + q;
              if (m < M) {
                const float y = FP8 ? acc[t][q] + b : fmaf(acc[t][q], ws2, b);
                Y[static_cast<size_t>(m) * N + n] = round_to<T>(y);
              }
            }
        }
      }
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    cp.advance(nws, stride);
  };

  for (int f0 = 0; f0 < total; f0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      load(raw[(u + D) % S]);
      if (f0 + u < total) consume(raw[u]);
    }
  }
}

// --------------------------------------------------------------------- launch

// Windows in flight per wave: the activation bytes of a slot grow with the
// row tiles, so the depth shrinks to stay within 256 registers.
template <int MT>
constexpr int sk_depth() {
  return MT == 1 ? 4 : (MT == 2 ? 3 : 1);
}

template <bool FP8, int MT>
constexpr size_t sk_lds() {
  return static_cast<size_t>(kSkWaves) * sk_lds_per_wave<FP8, sk_depth<MT>()>();
}

// Dynamic LDS above 64 KiB must be allowed per kernel, once per device.
template <typename T, bool FP8, int MT, int KS>
void sk_allow_lds() {
  static std::once_flag once[kMaxDevices];
  once_per_device(once, [] {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&skinny_kernel<T, FP8, MT, KS, sk_depth<MT>()>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sk_lds<FP8, MT>()));
  });
}

template <typename T, bool FP8, int MT, int KS>
int sk_slots() {
  sk_allow_lds<T, FP8, MT, KS>();
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, skinny_kernel<T, FP8, MT, KS, sk_depth<MT>()>,
                                                   64 * kSkWaves, sk_lds<FP8, MT>()) != hipSuccess ||
      v < 1)
    v = 1;
  return v * device_cus();
}

struct SkPlan {
  int KS, grid, nws;
};

// The K split KS (TPW = 8 / KS tiles side by side) with the least work on
// the busiest wave: rounds of tile groups per workgroup (persistent grid,
// capped at the resident workgroups) times windows per wave, counting the
// windows a wave pads with (FP4 waves start at even windows, since a weight
// unit holds two).  Ties go to less padding, then to the larger split; every
// wave keeps at least two windows.
template <typename T, bool FP8, int MT>
int sk_slots_ks(int ks) {
  switch (ks) {
    case 1: return sk_slots<T, FP8, MT, 1>();
    case 2: return sk_slots<T, FP8, MT, 2>();
    case 4: return sk_slots<T, FP8, MT, 4>();
    default: return sk_slots<T, FP8, MT, 8>();
  }
}

template <typename T, bool FP8, int MT>
SkPlan sk_plan(int64_t N, int NW) {
  const int64_t tiles = (N + 15) / 16;
  SkPlan best{1, 1, NW + (FP8 ? 0 : (NW & 1))};
  int64_t best_cost = -1;
  int best_pad = 0;
  for (int ks = kSkWaves; ks >= 1; ks >>= 1) {
    if (ks > 1 && NW < 2 * ks) continue;
    int nws = (NW + ks - 1) / ks;
    if (!FP8) nws += nws & 1;
    const int64_t ntg = (tiles + kSkWaves / ks - 1) / (kSkWaves / ks);
    const int64_t slots = sk_slots_ks<T, FP8, MT>(ks);
    const int64_t grid = ntg < slots ? ntg : slots;
    const int64_t cost = (ntg + grid - 1) / grid * nws;
    const int pad = nws * ks - NW;
    if (best_cost < 0 || cost < best_cost || (cost == best_cost && pad < best_pad)) {
      best_cost = cost;
      best_pad = pad;
      best = SkPlan{ks, static_cast<int>(grid), nws};
    }
  }
  return best;
}

// One plan per shape (occupancy queries cost more than the kernel).
struct SkEntry {
  int64_t N;
  int NW, MT, dev, kind;
  SkPlan p;
};

template <typename T, bool FP8, int MT>
SkPlan sk_cached_plan(int64_t N, int NW) {
  constexpr int kEntries = 64;
  static SkEntry table[kEntries];
  static int used = 0, next = 0;
  static std::mutex mu;
  const int kind = (FP8 ? 2 : 0) + (__is_same(T, __bf16) ? 1 : 0);
  int dev = 0;
  (void)hipGetDevice(&dev);
  {
    std::lock_guard<std::mutex> lock(mu);
    for (int i = 0; i < used; ++i) {
      const SkEntry& e = table[i];
      if (e.N == N && e.NW == NW && e.MT == MT && e.dev == dev && e.kind == kind) return e.p;
    }
  }
  const SkPlan p = sk_plan<T, FP8, MT>(N, NW);
  std::lock_guard<std::mutex> lock(mu);
  table[next] = SkEntry{N, NW, MT, dev, kind, p};
  next = (next + 1) % kEntries;
  if (used < kEntries) ++used;
  return p;
}

template <typename T, bool FP8, int MT>
void sk_launch_mt(const MatmulArgs& a, FastDiv wpb) {
  const int NW = static_cast<int>(a.K / 128);
  const SkPlan p = sk_cached_plan<T, FP8, MT>(a.N, NW);
  const int tiles = static_cast<int>((a.N + 15) / 16);
  hipStream_t s = static_cast<hipStream_t>(a.stream);
#define FP4W_SK_LAUNCH(KS_)                                                                              \
  sk_allow_lds<T, FP8, MT, KS_>();                                                                       \
  hipLaunchKernelGGL((skinny_kernel<T, FP8, MT, KS_, sk_depth<MT>()>), dim3(p.grid), dim3(64 * kSkWaves), \
                     (sk_lds<FP8, MT>()), s, static_cast<const T*>(a.A), a.B, a.scales, a.ws2, static_cast<const T*>(a.bias), \
                     static_cast<T*>(a.Y), static_cast<int>(a.M), static_cast<int>(a.N),                 \
                     static_cast<int>(a.K), static_cast<int>(a.scale_cols), wpb, tiles, p.nws)
  switch (p.KS) {
    case 1: FP4W_SK_LAUNCH(1); break;
    case 2: FP4W_SK_LAUNCH(2); break;
    case 4: FP4W_SK_LAUNCH(4); break;
    default: FP4W_SK_LAUNCH(8); break;
  }
#undef FP4W_SK_LAUNCH
}

template <typename T, bool FP8>
int sk_launch_t(const MatmulArgs& a) {
  // 32-bit buffer offsets: one 16-column tile and the activations must fit
  if (a.N > 0x7fffffff - 16 || a.K > (int64_t(1) << 26) || a.M * a.K * 2 >= (int64_t(1) << 31)) return -1;
  const FastDiv wpb = make_fastdiv(FP8 ? static_cast<uint32_t>(a.block_size / 128) : 1u);
  if (a.M <= 16)
    sk_launch_mt<T, FP8, 1>(a, wpb);
  else if (a.M <= 32)
    sk_launch_mt<T, FP8, 2>(a, wpb);
  else
    sk_launch_mt<T, FP8, 4>(a, wpb);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_fp4_skinny(const MatmulArgs& a) {
  return a.act == Act::BF16 ? sk_launch_t<__bf16, false>(a) : sk_launch_t<_Float16, false>(a);
}

int launch_fp8_skinny(const MatmulArgs& a) {
  return a.act == Act::BF16 ? sk_launch_t<__bf16, true>(a) : sk_launch_t<_Float16, true>(a);
}

}  // namespace fp4w

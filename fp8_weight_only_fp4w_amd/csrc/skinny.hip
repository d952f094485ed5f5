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
// covers k = 128 w .. 128 w + 127; MFMA step i of it takes the 32 k at
// 128 w + 32 i, lane group g = lane / 16 supplying 8 of them (the natural
// MFMA order).  The weights keep their 16-byte contiguous loads (64
// contiguous bytes per column and load instruction) and are moved between
// lane groups in registers, with v_permlane32_swap / v_permlane16_swap:
// each swaps one bit of the lane-group index with one bit of the register
// index.
//  * FP4: lane group s loads the 32 k at 128 w + 32 s, dwords d = 8-k units
//    4 s + d; swapping both lane-group bits with both register bits leaves
//    register i of group g holding unit 4 i + g, i.e. k 128 w + 32 i + 8 g.
//    That lane needs the scales of blocks 8 w + 2 i + g / 2, read as the
//    window's 8 scale bytes.
//  * FP8: lane group s loads k 128 w + 16 s .. + 15 and 128 w + 64 + 16 s ..
//    + 15 (8-k units 2 s, 2 s + 1, 8 + 2 s, 9 + 2 s); one swap of the high
//    lane-group bit with the low unit-slot bit leaves step i of group g with
//    unit 4 i + tau(g), tau(g) = 2 (g & 1) + (g >> 1).  The activations are
//    loaded with the same tau.
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
// scratch (16-byte chunks XOR-swizzled by row, conflict-free on both the
// write and the read side), which also holds the K-split reduction at the
// end of a tile.
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

// One window of one lane: weights, the block scale(s) of the lane's column,
// the bias bits (first window of a tile only) and 4 x 16 activation bytes per
// row tile (row-major: load q of tile t holds rows 16 t + 4 q .. + 3).
template <bool FP8, int MT>
struct SkRaw;
template <int MT>
struct SkRaw<false, MT> {
  u32x4 w;
  u32x2 sc;  // the 8 E4M3 scale bytes of the window
  uint32_t bias;
  u32x4 a[4 * MT];
};
template <int MT>
struct SkRaw<true, MT> {
  u32x4 w0, w1;
  uint32_t sc;  // FP32 block scale bits
  uint32_t bias;
  u32x4 a[4 * MT];
};

// v_permlane32_swap: the upper 32 lanes of a trade places with the lower 32
// lanes of b.  v_permlane16_swap: the odd 16-lane rows of a trade places
// with the even rows of b.
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}
__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
  a = r[0];
  b = r[1];
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
  typedef SkRaw<FP8, MT> RawT;
  typedef ActTraits<T> Tr;
  typedef typename Tr::vec8 V;
  // per wave: MT x 16 rows x 256 bytes of activations (one window), reused
  // for the K-split partial sums at the end of a tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int ks = wave % KS, tw = wave / KS;
  unsigned char* scr = smem + wave * (MT * 4096);
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
  // LDS byte offsets: row-major chunk written by this lane (load q adds
  // 1024 q and XORs the chunk with 4 q), and the chunk this lane reads for
  // MFMA step i (row li, chunk 4 i + tau(g); step i XORs with 4 i)
  const uint32_t tau = FP8 ? static_cast<uint32_t>(2 * (g & 1) + (g >> 1)) : static_cast<uint32_t>(g);
  const uint32_t w_lds = static_cast<uint32_t>(g) * 256u + 16u * static_cast<uint32_t>(li ^ g);
  const uint32_t r_lds = static_cast<uint32_t>(li) * 256u + 16u * (tau ^ static_cast<uint32_t>(li));
  // FP4: bit offset of the scale bytes of blocks 2 i + g / 2 in the window's
  // scale dwords (byte g / 2 for steps 0 and 2, byte 2 + g / 2 for 1 and 3)
  const uint32_t sc_shift = 8u * static_cast<uint32_t>(g >> 1);
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

  auto load = [&](RawT& r) {
    if (lp.j == 0) r.bias = buf_load_u16(biasr, 2u * li);
    const int w = ks * nws + lp.j;
    const bool ok = w < NW;  // windows past K read zeros (weights, scales, activations)
    if constexpr (FP8) {
      const uint32_t off = ok ? li * row_bytes + 128u * w + 16u * g : kOutOfRange;
      r.w0 = buf_load_b128(br, off);
      r.w1 = buf_load_b128(br, off + 64u);
      r.sc = buf_load_b32(sr, ok ? li * srow_bytes + 4u * scol(w) : kOutOfRange);
    } else {
      r.w = buf_load_b128(br, ok ? li * row_bytes + 64u * w + 16u * g : kOutOfRange);
      r.sc = buf_load_b64(sr, ok ? li * srow_bytes + 8u * w : kOutOfRange);
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

#pragma unroll
  for (int d = 0; d < D; ++d) load(raw[d]);

  auto consume = [&](const RawT& r) {
    const int j = cp.j;
    if (j == 0) tbias = r.bias;
    // activations: row-major chunks into the scratch, back in the MFMA
    // layout (same wave, so LDS order needs no wait between the two)
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<u32x4*>(scr + 4096 * t + 1024 * q + (w_lds ^ (64u * q))) = r.a[4 * t + q];
    V av[MT][4];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[t][i] = *reinterpret_cast<const V*>(scr + 4096 * t + (r_lds ^ (64u * i)));
    V bw[4];
    if constexpr (FP8) {
      // units 2s / 2s+1 (and 8+2s / 9+2s) of lane group s: swap the high
      // lane-group bit with the unit-slot bit
      uint32_t q[8] = {r.w0.x, r.w0.y, r.w0.z, r.w0.w, r.w1.x, r.w1.y, r.w1.z, r.w1.w};
      swap32(q[0], q[2]);
      swap32(q[1], q[3]);
      swap32(q[4], q[6]);
      swap32(q[5], q[7]);
      bw[0] = Tr::decode8_fp8(q[0], q[1]);
      bw[1] = Tr::decode8_fp8(q[2], q[3]);
      bw[2] = Tr::decode8_fp8(q[4], q[5]);
      bw[3] = Tr::decode8_fp8(q[6], q[7]);
      const float sc = __builtin_bit_cast(float, r.sc);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        f32x4 blk = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < 4; ++i) blk = Tr::mfma(av[t][i], bw[i], blk);
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = fmaf(blk[q], sc, acc[t][q]);
      }
    } else {
      // 4 x 4 transpose of dwords across lane groups: register i of group g
      // becomes k 32 i + 8 g of the window
      uint32_t q[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
      swap32(q[0], q[2]);
      swap32(q[1], q[3]);
      swap16(q[0], q[1]);
      swap16(q[2], q[3]);
      // scale of block 2 i + g / 2 for step i, folded into the operand
      const uint32_t lo = r.sc.x >> sc_shift, hi = r.sc.y >> sc_shift;
      bw[0] = Tr::decode8(q[0], Tr::make_scale(e4m3_to_f32<0>(lo)));
      bw[1] = Tr::decode8(q[1], Tr::make_scale(e4m3_to_f32<2>(lo)));
      bw[2] = Tr::decode8(q[2], Tr::make_scale(e4m3_to_f32<0>(hi)));
      bw[3] = Tr::decode8(q[3], Tr::make_scale(e4m3_to_f32<2>(hi)));
#pragma unroll
      for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[t] = Tr::mfma(av[t][i], bw[i], acc[t]);
    }
    if (j == nws - 1) {
      // end of a tile: reduce the K split through LDS, then the epilogue
      if (KS > 1) {
        // partial sums in the first MT KiB of each wave's scratch (its reads
        // of this window were issued before these writes)
        f32x4* red = reinterpret_cast<f32x4*>(smem);
        constexpr int kWaveVec = MT * 4096 / 16;  // f32x4 per wave scratch
#pragma unroll
        for (int t = 0; t < MT; ++t) red[wave * kWaveVec + t * 64 + lane] = acc[t];
        __syncthreads();
        if (ks == 0) {
#pragma unroll
          for (int v = 1; v < KS; ++v)
#pragma unroll
            for (int t = 0; t < MT; ++t) acc[t] += red[(wave + v) * kWaveVec + t * 64 + lane];
        }
        __syncthreads();
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

int sk_num_cus() {
  static int cus = -1;
  if (cus < 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1)
      v = 256;
    cus = v;
  }
  return cus;
}

template <int MT>
constexpr size_t sk_lds() {
  return static_cast<size_t>(kSkWaves) * MT * 4096;
}

// Dynamic LDS above 64 KiB must be allowed per kernel, once.
template <typename T, bool FP8, int MT, int KS>
void sk_allow_lds() {
  static bool done = false;
  if (!done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&skinny_kernel<T, FP8, MT, KS, sk_depth<MT>()>),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(sk_lds<MT>()));
    done = true;
  }
}

template <typename T, bool FP8, int MT, int KS>
int sk_slots() {
  sk_allow_lds<T, FP8, MT, KS>();
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, skinny_kernel<T, FP8, MT, KS, sk_depth<MT>()>,
                                                   64 * kSkWaves, sk_lds<MT>()) != hipSuccess ||
      v < 1)
    v = 1;
  return v * sk_num_cus();
}

struct SkPlan {
  int KS, grid, nws;
};

template <typename T, bool FP8, int MT>
SkPlan sk_plan(int64_t N, int NW) {
  const int64_t tiles = (N + 15) / 16;
  int ks = kSkWaves;
  while (ks > 1 && NW < 2 * ks) ks >>= 1;  // at least two windows per wave
  int slots = 0;
  switch (ks) {
    case 1: slots = sk_slots<T, FP8, MT, 1>(); break;
    case 2: slots = sk_slots<T, FP8, MT, 2>(); break;
    case 4: slots = sk_slots<T, FP8, MT, 4>(); break;
    default: slots = sk_slots<T, FP8, MT, 8>(); break;
  }
  const int64_t ntg = (tiles + kSkWaves / ks - 1) / (kSkWaves / ks);
  return SkPlan{ks, static_cast<int>(ntg < slots ? ntg : slots), (NW + ks - 1) / ks};
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
                     sk_lds<MT>(), s, static_cast<const T*>(a.A), a.B, a.scales, a.ws2, static_cast<const T*>(a.bias), \
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

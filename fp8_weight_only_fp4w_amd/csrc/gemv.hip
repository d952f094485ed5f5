// Decode GEMV (1 <= M <= 8) for weight-only FP4 and FP8, on MFMA.
//
// Memory-bound: every packed weight byte and scale byte is read from HBM once
// with 16-byte loads; activations (M x K, at most a few hundred KiB) come from
// LDS or L2.
//
// Common structure (the pages' CUDA version is [FP4 doc] §4 "Tensor-core
// sub-path" / [FP8 doc] §4.1, with mma.m16n8k16; this is re-derived for the
// CDNA4 MFMA layouts).  A wave owns a tile of 16 output columns n (the MFMA B
// operand: lane l supplies column l % 16).  K is a reduction axis, so it is
// permuted freely as long as both operands agree: in window w (128 k) lane
// group g = l / 16 loads the contiguous chunk c = 4w + g of 32 k of its
// column, one 16-byte load per lane for FP4 (two for FP8).
//
// FP4 (16x16x32 MFMA, "block-diagonal" activations).  Folding the E4M3 scale
// into BF16 weights would be exact ([FP4 doc] §4), but costs a convert, two
// FP32 multiplies and a pack per pair of weights, which makes a wave64 GEMV
// VALU-bound on CDNA4.  Instead the weights are converted unscaled (one
// instruction per pair) and every 16-k scale block gets its own FP32 dot,
// scaled by its E4M3 value with one FMA.  Four blocks share each MFMA: lane
// group g holds blocks 2g and 2g + 1 of the window, so in MFMA (s, p) the
// four lane groups supply piece p (8 k) of blocks 2g + s, g = 0..3.  Row
// i = 4 m' + q of the A operand carries activation row m = m' (+ 4 for the
// second row half) in the k slots of lane group q only, and zeros elsewhere;
// summing the two pieces p therefore leaves in result row (m', q) the full
// dot of row m with block 2q + s.  The result lane (column n, group g) holds
// rows 4g .. 4g + 3 = the four blocks of one activation row, so a window
// costs 4 MFMAs and 8 FMAs per row half, with no data exchange between lanes.
// weight_scale_2 and the bias are applied once in the epilogue.
//
// FP8 (16x16x32 MFMA).  E4M3 -> T is exact and the FP32 block scale is
// applied to a window (128 k, inside one scale block: block_size % 128 == 0)
// accumulated in a fresh MFMA accumulator.  Result lane (n, g) holds rows
// 4g .. 4g + 3.
//
// Latency hiding (what decides the bandwidth): a wave keeps D windows of
// weights in flight ahead of the one it multiplies; the pipeline runs as one
// flat sequence over all tile groups the (persistent) workgroup owns, so it
// never drains between tiles.  All loads are raw buffer loads and
// branch-free (tails read zeros), so the loop only ever waits for its oldest
// load.  A workgroup is KS x TPW waves: KS waves split the K windows of one
// tile (the page's KSplit, reduced through LDS), TPW tiles side by side.
//
// [FP4 doc] = "MatMulBlockQuantizedFp4Weight - CUDA Operator Documentation"
// [FP8 doc] = "MatMulBlockQuantizedFp8Weight - CUDA Operator Documentation"

#include <hip/hip_runtime.h>

#include <mutex>

#include "device.h"
#include "launch.h"

namespace fp4w {
namespace {

constexpr int kWaves = 8;  // waves per workgroup (KS x TPW)

// Raw data of one window for one lane.  FP4: 16 weight bytes; FP8: 32.  The
// block scales of a tile are read in 64-byte pieces per column (one request
// per row instead of one per row and window): the piece rides along with the
// first window of each group of kScaleWin windows and is parked in a per-wave
// LDS slice, from which every window of the group reads its scales.  The bias
// bits of the lane's column ride along with the first window of a tile.
// Activations ride along only when they come from L2 (ACT_REG).
template <bool FP8, bool ACT_REG, int R>
struct Raw;
template <bool ACT_REG, int R>
struct Raw<false, ACT_REG, R> {
  u32x4 w;
  u32x4 sc;
  uint32_t bias;
  u32x4 a[ACT_REG ? 4 * R : 1];  // 64 activation bytes per row half
};
template <bool ACT_REG, int R>
struct Raw<true, ACT_REG, R> {
  u32x4 w0, w1;
  u32x4 sc;
  uint32_t bias;
  u32x4 a[ACT_REG ? 4 : 1];  // 4 x 8 activations
};

// Windows per 64-byte scale piece: FP4 has 8 E4M3 bytes per window, FP8 one
// FP32 scale per 128-k window (or per several windows: block_size % 128 == 0,
// and 16 consecutive columns always cover 16 consecutive windows).
template <bool FP8>
constexpr int kScaleWin = FP8 ? 16 : 8;

// Position of a wave in its flat window sequence: tile group and window.
struct Pos {
  int tg, j;
  __device__ __forceinline__ void advance(int nws, int stride) {
    if (++j == nws) {
      j = 0;
      tg += stride;
    }
  }
};

// Activations, two ways (ACT_LDS):
//  * false: loaded from L2 with the weights, at the same pipeline depth;
//  * true: copied once into LDS by the persistent workgroup (rows zero-padded
//    to whole 128-k windows; for FP4 a 256-byte zero block follows the M rows
//    and serves the lanes that carry no row), so the loop issues weight loads
//    only.
// Either way the load consumed next is always the oldest one in flight.
// R: FP4 - row halves (1: M <= 4, 2: M <= 8); FP8 - result rows a lane
// scales (1, 2 or 4).  D: windows in flight ahead of the multiply.
//
// LDS: [kWaves][1 KiB] per-wave slices (scale pieces, and the K-split
// reduction at the end of a tile), then the activation rows.
template <typename T, int KS, bool FP8, bool ACT_LDS, int R, int D>
__global__ __launch_bounds__(64 * kWaves) void gemv_kernel(
    const T* __restrict__ A, const uint8_t* __restrict__ B, const void* __restrict__ scales,
    const float* __restrict__ ws2p, const T* __restrict__ bias, T* __restrict__ Y, int M, int N,
    int K, int cols, FastDiv win_per_block, FastDiv chunks_per_row, int num_tiles, int nws) {
  constexpr bool ACT_REG = !ACT_LDS;
  constexpr int TPW = kWaves / KS;
  constexpr int S = D + 1;  // register slots of the pipeline
  constexpr int SW = kScaleWin<FP8>;
  typedef Raw<FP8, ACT_REG, R> RawT;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int li = lane & 15, g = lane >> 4;
  const int ks = wave % KS, tw = wave / KS;
  const int NW = K >> 7;  // 128-k windows (K % 128 == 0)
  const int ntg = (num_tiles + TPW - 1) / TPW;
  const int iters = (ntg - static_cast<int>(blockIdx.x) + static_cast<int>(gridDim.x) - 1) /
                    static_cast<int>(gridDim.x);
  // every wave of the workgroup runs the same sequence, so the barriers of
  // the K-split reduction are uniform
  const int total = iters * nws;
  const int stride = gridDim.x;
  const uint32_t row_bytes = FP8 ? static_cast<uint32_t>(K) : static_cast<uint32_t>(K >> 1);
  const uint32_t srow_bytes = FP8 ? static_cast<uint32_t>(cols) * 4u : static_cast<uint32_t>(cols);
  const float ws2 = FP8 ? 1.0f : *ws2p;  // one scalar load, kept in a register

  f32x4* red = reinterpret_cast<f32x4*>(smem);       // [kWaves][64]
  unsigned char* slice = smem + 1024 * wave;          // this wave's 1 KiB
  unsigned char* a_lds = smem + kWaves * 1024;
  const uint32_t lds_pitch = static_cast<uint32_t>(NW) * 256u + 16u;  // bytes per LDS row of A
  const uint32_t zero_off = static_cast<uint32_t>(M) * lds_pitch;       // FP4: the zero block
  const uint32_t a_bytes = static_cast<uint32_t>(M) * static_cast<uint32_t>(K) * 2u;
  const rsrc_t a_rsrc = make_rsrc(A, a_bytes);

  // Per-lane activation offsets (bytes, window 0).  FP4: lane (li = 4m' + q,
  // g) carries row m = m' + 4h of half h when q == g, else zeros (the zero
  // block in LDS, or an out-of-range offset).  FP8: row li (rows >= M are
  // never stored, so lanes li >= M may read any valid row).
  uint32_t a_off[FP8 ? 1 : R];
  bool a_valid[FP8 ? 1 : R];
  if constexpr (FP8) {
    a_off[0] = ACT_LDS ? static_cast<uint32_t>(li % M) * lds_pitch
                       : static_cast<uint32_t>(li) * static_cast<uint32_t>(K) * 2u;
  } else {
#pragma unroll
    for (int h = 0; h < R; ++h) {
      const int m = (li >> 2) + 4 * h;
      const bool valid = (li & 3) == g && m < M;
      a_valid[h] = valid;
      if constexpr (ACT_LDS)
        a_off[h] = static_cast<uint32_t>(valid ? m : 0) * lds_pitch + 64u * g;
      else
        a_off[h] = valid ? static_cast<uint32_t>(m) * static_cast<uint32_t>(K) * 2u + 64u * g : kOutOfRange;
    }
  }
  // scale column of window w (FP8; windows past NW are clamped)
  auto scol = [&](int w) {
    return min(fdiv(static_cast<uint32_t>(min(w, NW - 1)), win_per_block), static_cast<uint32_t>(cols - 1));
  };

  // Window mapping.  FP4: lane group g loads the 32 k of chunk c = 4w + g
  // (bytes 64w + 16g of its column: one wave instruction reads 64 contiguous
  // bytes of each of 16 rows).  FP8: lane group g loads k 128w + 16g .. + 15
  // and 128w + 64 + 16g .. + 15 (two instructions, each 64 contiguous bytes
  // per row).
  // Load side of the pipeline: position and the (wave-uniform) descriptors
  // of its tile, recomputed only when the position enters a new tile.
  Pos lp{static_cast<int>(blockIdx.x), 0};  // next window to load
  rsrc_t br, sr, biasr;
  auto set_load_tile = [&]() {
    const int t = lp.tg * TPW + tw;
    const int rows = max(0, min(16, N - 16 * t));
    const size_t n0 = static_cast<size_t>(16) * t;
    br = make_rsrc(B + n0 * row_bytes, rows * row_bytes);
    sr = make_rsrc(static_cast<const uint8_t*>(scales) + n0 * srow_bytes, rows * srow_bytes);
    biasr = make_rsrc(bias + n0, bias ? rows * 2u : 0u);
  };
  set_load_tile();
  // per-lane byte offsets of the lane's column (window 0); the window's own
  // offset is wave-uniform and rides in the scalar offset of the load.  Lanes
  // past the tile's last row are out of range through their own offset.
  const uint32_t w_lane = li * row_bytes + 16u * g;

  auto load = [&](RawT& r) {
    // bias and scale pieces are only requested for the windows that carry
    // them (uniform branches; an out-of-range request would still occupy the
    // load pipeline for all 64 lanes)
    if (lp.j == 0) r.bias = buf_load_u16(biasr, 2u * li);
    const int w = ks * nws + lp.j;
    const bool ok = w < NW;
    const bool piece = ok && lp.j % SW == 0;
    if constexpr (FP8) {
      const uint32_t off = ok ? li * row_bytes + 128u * w + 16u * g : kOutOfRange;
      r.w0 = buf_load_b128(br, off);
      r.w1 = buf_load_b128(br, off + 64u);
      // FP32 scales of columns scol(w) .. + 15 (bytes past the row are never used)
      if (piece) r.sc = buf_load_b128(sr, li * srow_bytes + 4u * scol(w) + 16u * g);
      if constexpr (ACT_REG) {
        const uint32_t aoff = ok ? a_off[0] + 256u * w + 32u * g : kOutOfRange;
        r.a[0] = buf_load_b128(a_rsrc, aoff);
        r.a[1] = buf_load_b128(a_rsrc, aoff + 16u);
        r.a[2] = buf_load_b128(a_rsrc, aoff + 128u);
        r.a[3] = buf_load_b128(a_rsrc, aoff + 144u);
      }
    } else {
      // windows past NW re-read window NW - 1 (inside the row) and are
      // cancelled by zero scales when multiplied
      r.w = buf_load_b128_so(br, w_lane, 64u * static_cast<uint32_t>(min(w, NW - 1)));
      // E4M3 scales of windows w .. w + 7 (bytes past the row are never used)
      if (piece) r.sc = buf_load_b128(sr, li * srow_bytes + 8u * w + 16u * g);
      if constexpr (ACT_REG) {
#pragma unroll
        for (int h = 0; h < R; ++h) {
          // out-of-range lanes stay out of range: a_off < 2^31 or >= 2^31
          const uint32_t aoff = ok ? a_off[h] + 256u * w : kOutOfRange;
#pragma unroll
          for (int i = 0; i < 4; ++i) r.a[4 * h + i] = buf_load_b128(a_rsrc, aoff + 16u * i);
        }
      }
    }
    if (++lp.j == nws) {
      lp.j = 0;
      lp.tg += stride;
      set_load_tile();
    }
  };

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  uint32_t tbias = 0;  // bias bits of the lane's column, current tile
  RawT raw[S];
  Pos cp{static_cast<int>(blockIdx.x), 0};  // window being multiplied

  if constexpr (ACT_LDS) {
    // Rows 0 .. M-1 of A, zero beyond K, then (FP4) the zero row.  The first
    // eight 16-byte chunks per thread are requested before the weights, so
    // their stores wait for them alone (loads complete in order); any further
    // chunks (large M x K) follow the weight requests.  Chunk indices past the
    // end are clamped to the last chunk (same data, same address), so every
    // load is consumed by a store and none stays in flight into the main loop.
    const uint32_t cpr = chunks_per_row.d;  // lds_pitch / 16
    const uint32_t nload = static_cast<uint32_t>(M) * cpr;
    const uint32_t nall = FP8 ? nload : nload + 16u;  // FP4: the 256-byte zero block
    constexpr uint32_t kStep = 64u * kWaves;
    auto fill_load = [&](uint32_t q0, u32x4 (&v)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t q = min(q0 + i * kStep, nload - 1u);
        const uint32_t row = fdiv(q, chunks_per_row), col = q - row * cpr;
        const uint32_t off = col * 8u < static_cast<uint32_t>(K) ? row * static_cast<uint32_t>(K) * 2u + col * 16u
                                                                : kOutOfRange;
        v[i] = buf_load_b128(a_rsrc, off);
      }
    };
    auto fill_store = [&](uint32_t q0, const u32x4 (&v)[8]) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        *reinterpret_cast<u32x4*>(a_lds + 16u * min(q0 + i * kStep, nload - 1u)) = v[i];
    };
    u32x4 v[8];
    fill_load(threadIdx.x, v);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load(raw[d]);
    }
    fill_store(threadIdx.x, v);
    for (uint32_t q0 = threadIdx.x + 8u * kStep; q0 < nload; q0 += 8u * kStep) {
      fill_load(q0, v);
      fill_store(q0, v);
    }
    for (uint32_t q = nload + threadIdx.x; q < nall; q += kStep)
      *reinterpret_cast<u32x4*>(a_lds + 16u * q) = u32x4{0u, 0u, 0u, 0u};
    __syncthreads();
  } else {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      load(raw[d]);
    }
  }

  // multiply one window (and finish its tile group after the last window)
  auto consume = [&](const RawT& r) {
    const int j = cp.j;
    const int w = min(ks * nws + j, NW - 1);  // windows past NW meet zero weights
    if (j % SW == 0) *reinterpret_cast<u32x4*>(slice + 64 * li + 16 * g) = r.sc;
    if (j == 0) tbias = r.bias;
    if constexpr (FP8) {
      typedef ActTraits<T> Tr;
      typedef typename Tr::vec8 V;
      // the scale of this window's column, from the piece of the first
      // window of its group (the column offset is at most 15)
      const uint32_t c0 = scol(ks * nws + (j - j % SW));
      const float sc = *reinterpret_cast<const float*>(slice + 64 * li + 4 * (scol(w) - c0));
      V a[4];
      if constexpr (ACT_LDS) {
        const unsigned char* q = a_lds + a_off[0] + 256u * w + 32u * g;
        a[0] = *reinterpret_cast<const V*>(q);
        a[1] = *reinterpret_cast<const V*>(q + 16u);
        a[2] = *reinterpret_cast<const V*>(q + 128u);
        a[3] = *reinterpret_cast<const V*>(q + 144u);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(V, r.a[i]);
      }
      f32x4 blk = f32x4{0.f, 0.f, 0.f, 0.f};
      blk = Tr::mfma(a[0], Tr::decode8_fp8(r.w0.x, r.w0.y), blk);
      blk = Tr::mfma(a[1], Tr::decode8_fp8(r.w0.z, r.w0.w), blk);
      blk = Tr::mfma(a[2], Tr::decode8_fp8(r.w1.x, r.w1.y), blk);
      blk = Tr::mfma(a[3], Tr::decode8_fp8(r.w1.z, r.w1.w), blk);
      // lane holds column n (one scale) and rows 4g .. 4g + 3
#pragma unroll
      for (int i = 0; i < R; ++i) acc[i] = fmaf(blk[i], sc, acc[i]);
    } else {
      typedef ActTraits<T> Tr;
      typedef typename Tr::vec8 V;
      // windows past NW (re-reads of window NW - 1) contribute nothing
      const u32x2 sb = ks * nws + j < NW ? *reinterpret_cast<const u32x2*>(slice + 64 * li + 8 * (j % SW))
                                          : u32x2{0u, 0u};
      // activations of the lane: 4 x 16 bytes per row half; chunk i = 2s + p
      // holds k 32g + 16s + 8p .. + 7 of the window (piece p of set s)
      u32x4 av[R][4];
#pragma unroll
      for (int h = 0; h < R; ++h) {
        if constexpr (ACT_LDS) {
          const unsigned char* q = a_lds + (a_valid[h] ? a_off[h] + 256u * w : zero_off);
#pragma unroll
          for (int i = 0; i < 4; ++i) av[h][i] = *reinterpret_cast<const u32x4*>(q + 16u * i);
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) av[h][i] = r.a[4 * h + i];
        }
      }
      // weights of piece p of set s (block 2g + s): dword 2s + p (8 codes)
      V bw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) bw[i] = Tr::decode8_fp4(r.w[i]);
      const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
      f32x4 d[R][2];
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          d[h][s] = Tr::mfma(__builtin_bit_cast(V, av[h][2 * s]), bw[2 * s], zero);
          d[h][s] = Tr::mfma(__builtin_bit_cast(V, av[h][2 * s + 1]), bw[2 * s + 1], d[h][s]);
        }
      // result row r of set s is block 2r + s: scale byte 2r + s
      const f32x2 s01 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(sb.x), false);
      const f32x2 s23 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(sb.x), true);
      const f32x2 s45 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(sb.y), false);
      const f32x2 s67 = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(sb.y), true);
      const float sc[8] = {s01.x, s01.y, s23.x, s23.y, s45.x, s45.y, s67.x, s67.y};
#pragma unroll
      for (int h = 0; h < R; ++h)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
#pragma unroll
          for (int s = 0; s < 2; ++s) acc[h] = fmaf(d[h][s][rr], sc[2 * rr + s], acc[h]);
    }
    if (j == nws - 1) {
      // end of this tile group: reduce the K split (the slices are free: every
      // wave has read its scales for this window), then the epilogue (uniform
      // across the workgroup: every wave has the same sequence)
      if (KS > 1) {
        red[wave * 64 + lane] = acc;
        __syncthreads();
        if (ks == 0) {
#pragma unroll
          for (int v = 1; v < KS; ++v) acc += red[(wave + v) * 64 + lane];
        }
        __syncthreads();
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
              const int m = g + 4 * h;
              if (m < M) Y[static_cast<size_t>(m) * N + n] = round_to<T>(fmaf(acc[h], ws2, b));
            }
          }
        }
      }
      acc = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    cp.advance(nws, stride);
  };

  // Window f sits in slot f % S.  Loads run ahead unconditionally (past the
  // end they are out of range), so every step waits only for its own, oldest,
  // loads; steps past the end of the sequence skip the multiply (the
  // condition is uniform across the workgroup).
  for (int f0 = 0; f0 < total; f0 += S) {
#pragma unroll
    for (int u = 0; u < S; ++u) {
      load(raw[(u + D) % S]);
      if (f0 + u < total) consume(raw[u]);
    }
  }
}

// --------------------------------------------------------------------- launch

constexpr size_t kMaxLds = 160 * 1024;  // LDS per workgroup on gfx950

// Pipeline depth (windows in flight per wave), from measurement: FP4 with
// activations in LDS gains up to 5; FP8 loads twice the bytes per window and
// is best at 3.
template <bool FP8, bool ACT_LDS>
constexpr int depth() {
  return ACT_LDS && !FP8 ? 5 : 3;
}

size_t lds_bytes(bool act_lds, bool fp8, int M, int NW) {
  // FP4: the M rows plus the 256-byte zero block
  return kWaves * 1024 +
         (act_lds ? static_cast<size_t>(M) * (static_cast<size_t>(NW) * 256 + 16) + (fp8 ? 0 : 256) : 0);
}

int num_cus() {
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

template <typename T, int KS, bool FP8, bool ACT_LDS, int R>
constexpr auto kernel_ptr() {
  return &gemv_kernel<T, KS, FP8, ACT_LDS, R, depth<FP8, ACT_LDS>()>;
}

// Dynamic LDS above 64 KiB must be allowed per kernel, once.
template <typename T, int KS, bool FP8, bool ACT_LDS, int R>
void allow_lds() {
  static bool done = false;
  if (!done) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kernel_ptr<T, KS, FP8, ACT_LDS, R>()),
                              hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kMaxLds));
    done = true;
  }
}

// Resident workgroups per CU for a kernel variant and LDS size.
template <typename T, int KS, bool FP8, bool ACT_LDS, int R>
int wg_per_cu(size_t lds) {
  allow_lds<T, KS, FP8, ACT_LDS, R>();
  int v = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&v, kernel_ptr<T, KS, FP8, ACT_LDS, R>(), 64 * kWaves,
                                                   lds) != hipSuccess ||
      v < 1)
    v = 1;
  return v;
}

template <typename T, int KS, bool FP8, bool ACT_LDS>
int wg_per_cu_r(int R, size_t lds) {
  if (R == 1) return wg_per_cu<T, KS, FP8, ACT_LDS, 1>(lds);
  if (R == 2 || !FP8) return wg_per_cu<T, KS, FP8, ACT_LDS, 2>(lds);
  return wg_per_cu<T, KS, FP8, ACT_LDS, (FP8 ? 4 : 2)>(lds);
}

template <typename T, bool FP8, bool ACT_LDS>
int slots_for(int KS, int R, int M, int NW) {
  const size_t lds = lds_bytes(ACT_LDS, FP8, M, NW);
  int per = 1;
  switch (KS) {
    case 1: per = wg_per_cu_r<T, 1, FP8, ACT_LDS>(R, lds); break;
    case 2: per = wg_per_cu_r<T, 2, FP8, ACT_LDS>(R, lds); break;
    case 4: per = wg_per_cu_r<T, 4, FP8, ACT_LDS>(R, lds); break;
    default: per = wg_per_cu_r<T, 8, FP8, ACT_LDS>(R, lds); break;
  }
  return num_cus() * per;
}

struct Plan {
  int KS, grid, nws;
  bool act_lds;
};

// Launch plan (rules from measurements on the decode, FP8 and wide-output
// shapes).  Activations go to LDS whenever they fit (reading them from L2 per
// window costs more load instructions than the weights themselves).  Few
// tiles (fewer than two per CU): 4 waves split K and a workgroup owns two
// tiles, which halves the activation fill per tile; many tiles: 8 waves split
// K of one tile.  Each wave keeps at least two windows.  The grid is the
// number of tile groups, capped at the resident workgroups (persistent).
template <typename T, bool FP8>
Plan plan(int64_t N, int M, int R, int NW) {
  const int64_t tiles = (N + 15) / 16;
  const int cus = num_cus();
  const bool lds = lds_bytes(true, FP8, M, NW) <= kMaxLds;
  int ks = tiles < 2 * static_cast<int64_t>(cus) ? 4 : 8;
  while (ks > 1 && NW < 2 * ks) ks >>= 1;
  const int64_t ntg = (tiles + kWaves / ks - 1) / (kWaves / ks);
  const int64_t slots = lds ? slots_for<T, FP8, true>(ks, R, M, NW) : slots_for<T, FP8, false>(ks, R, M, NW);
  return Plan{ks, static_cast<int>(ntg < slots ? ntg : slots), (NW + ks - 1) / ks, lds};
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

template <typename T, int KS, bool FP8, bool LDS>
void launch_v(const MatmulArgs& a, const Plan& p, int R, size_t lds, FastDiv wpb, FastDiv cpr, int tiles) {
  hipStream_t s = static_cast<hipStream_t>(a.stream);
#define FP4W_GEMV_LAUNCH(R_)                                                                           \
  allow_lds<T, KS, FP8, LDS, R_>();                                                                    \
  hipLaunchKernelGGL((gemv_kernel<T, KS, FP8, LDS, R_, depth<FP8, LDS>()>), dim3(p.grid),              \
                     dim3(64 * kWaves), lds, s, static_cast<const T*>(a.A), a.B, a.scales, a.ws2,      \
                     static_cast<const T*>(a.bias), static_cast<T*>(a.Y), static_cast<int>(a.M),       \
                     static_cast<int>(a.N), static_cast<int>(a.K), static_cast<int>(a.scale_cols), wpb, \
                     cpr, tiles, p.nws)
  if (R == 1) {
    FP4W_GEMV_LAUNCH(1);
  } else if (R == 2) {
    FP4W_GEMV_LAUNCH(2);
  } else if constexpr (FP8) {
    FP4W_GEMV_LAUNCH(4);
  }
#undef FP4W_GEMV_LAUNCH
}

template <typename T, bool FP8>
int launch_t(const MatmulArgs& a) {
  // buffer offsets are 32-bit: one 16-column tile and the activations must fit
  if (a.N > 0x7fffffff - 16 || a.K > (int64_t(1) << 26) || a.M * a.K * 2 >= (int64_t(1) << 31))
    return -1;
  const int M = static_cast<int>(a.M);
  const int NW = static_cast<int>(a.K / 128);
  // FP8: result rows a lane scales; FP4: row halves
  const int R = FP8 ? (M >= 3 ? 4 : M) : (M > 4 ? 2 : 1);
  const Plan p = cached_plan<T, FP8>(a.N, M, R, NW);
  const int tiles = static_cast<int>((a.N + 15) / 16);
  const size_t lds = lds_bytes(p.act_lds, FP8, M, NW);
  const FastDiv wpb = make_fastdiv(FP8 ? static_cast<uint32_t>(a.block_size / 128) : 1u);
  const FastDiv cpr = make_fastdiv(static_cast<uint32_t>(NW) * 16u + 1u);  // 16-byte chunks per LDS row
#define FP4W_GEMV_KS(LDS_)                                                   \
  switch (p.KS) {                                                            \
    case 1: launch_v<T, 1, FP8, LDS_>(a, p, R, lds, wpb, cpr, tiles); break;  \
    case 2: launch_v<T, 2, FP8, LDS_>(a, p, R, lds, wpb, cpr, tiles); break;  \
    case 4: launch_v<T, 4, FP8, LDS_>(a, p, R, lds, wpb, cpr, tiles); break;  \
    default: launch_v<T, 8, FP8, LDS_>(a, p, R, lds, wpb, cpr, tiles); break; \
  }
  if (p.act_lds) {
    FP4W_GEMV_KS(true)
  } else {
    FP4W_GEMV_KS(false)
  }
#undef FP4W_GEMV_KS
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace

int launch_fp4_gemv(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_t<__bf16, false>(a) : launch_t<_Float16, false>(a);
}

int launch_fp8_gemv(const MatmulArgs& a) {
  return a.act == Act::BF16 ? launch_t<__bf16, true>(a) : launch_t<_Float16, true>(a);
}

}  // namespace fp4w

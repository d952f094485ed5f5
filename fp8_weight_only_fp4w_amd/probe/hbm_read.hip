// Read-stream probe: the measured HBM read rate that the decode GEMV is
// compared with.  Every 16-byte piece of a buffer is read once per launch by
// non-temporal 16-byte loads in a grid-stride loop, U pieces in flight per
// thread, and XOR-reduced per thread.  A thread stores its reduction only if
// it equals `key`, which the caller picks so that it never does for the data
// it fills in; the loads cannot be removed and nothing is written.
//
// A second kernel streams with the decode GEMV's load structure (below).
//
// This is measurement code, built into its own library (libhbmprobe.so); the
// matmul library does not use it.

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(512) void hbm_read_kernel(const u32x4* __restrict__ p, uint64_t n, uint32_t key,
                                                       uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const uint64_t stride = static_cast<uint64_t>(gridDim.x) * 512u * U;
  for (uint64_t i = static_cast<uint64_t>(blockIdx.x) * 512u * U + threadIdx.x; i < n; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      v[u] = i + u * 512u < n ? __builtin_nontemporal_load(p + i + u * 512u) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == key) sink[static_cast<size_t>(blockIdx.x) * 512u + threadIdx.x] = acc;
}

// The decode GEMV's load structure without its arithmetic: 8 waves per
// workgroup, each streaming units of 2 KiB (two 1 KiB direct-to-LDS loads)
// into a private ring of D + 1 slots with D units in flight, waiting for the
// oldest unit and reading one 16-byte chunk of it back per lane.  Unit i of
// wave w of the grid is the 2 KiB at (i * waves + w) * 2048.
template <int D>
__global__ __launch_bounds__(512) void lds_stream_kernel(const uint8_t* __restrict__ buf, uint32_t bytes, int units,
                                                         uint32_t key, uint32_t* __restrict__ sink) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t waves = gridDim.x * 8u, gw = blockIdx.x * 8u + wave;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), 0, bytes, 0x00020000);
  typedef __attribute__((address_space(3))) void* lds_ptr;
  unsigned char* ring = smem + wave * (D + 1) * 2048;
  // past the last unit the loads take an offset past the buffer: they read
  // nothing and write zeros into a slot no one reads
  auto issue = [&](int i, int slot) {
    const bool live = i < units;
    const uint32_t base = live ? (static_cast<uint32_t>(i) * waves + gw) * 2048u : 0u;
    const uint32_t v = live ? 16u * lane : 0x80000000u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(ring + slot * 2048), 16, v, base, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr)(ring + slot * 2048 + 1024), 16, live ? v + 1024u : v, base, 0, 0);
  };
  uint32_t acc = 0;
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);
  for (int i0 = 0; i0 < units; i0 += D + 1) {
#pragma unroll
    for (int s = 0; s < D + 1; ++s) {
      issue(i0 + s + D, (s + D) % (D + 1));
      // the oldest unit (this slot) has landed: 2 D loads may stay in flight
      __builtin_amdgcn_s_waitcnt(((2 * D) & 15) | (((2 * D) >> 4) << 14) | (0x7 << 4) | (0xF << 8));
      const uint32_t* q = reinterpret_cast<const uint32_t*>(ring + s * 2048 + 16 * lane);
      if (i0 + s < units) acc ^= q[0] ^ q[3];
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  if (acc == key) sink[static_cast<size_t>(blockIdx.x) * 512u + threadIdx.x] = acc;
}

}  // namespace

// buf: device buffer of `bytes` bytes (a multiple of 16); sink: device buffer
// of grid * 512 uint32 (written only where a thread's reduction equals key);
// grid: workgroups of 512 threads, 1 .. 65536; unroll: 4 or 8 pieces in
// flight per thread.  Enqueues one launch on `stream`; returns 0, -1 for bad
// arguments (nothing launched), -2 if the launch failed.
extern "C" int hbm_read_probe(const void* buf, uint64_t bytes, int grid, int unroll, uint32_t key, uint32_t* sink,
                              hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || bytes % 16 != 0 || grid < 1 || grid > 65536 ||
      (unroll != 4 && unroll != 8))
    return -1;
  const uint64_t n = bytes / 16;
  const u32x4* p = static_cast<const u32x4*>(buf);
  if (unroll == 4)
    hipLaunchKernelGGL(hbm_read_kernel<4>, dim3(grid), dim3(512), 0, stream, p, n, key, sink);
  else
    hipLaunchKernelGGL(hbm_read_kernel<8>, dim3(grid), dim3(512), 0, stream, p, n, key, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// The GEMV-structured stream above: `grid` workgroups of 8 waves, `units`
// units of 2 KiB per wave (buf holds at least grid * 8 * units * 2048 bytes,
// below 4 GiB), 4 units in flight per wave; sink and key as for
// hbm_read_probe.  Returns 0, -1 for bad arguments (nothing launched), -2 if
// the launch failed.
extern "C" int hbm_lds_stream_probe(const void* buf, uint64_t bytes, int grid, int units, uint32_t key, uint32_t* sink,
                                    hipStream_t stream) {
  if (buf == nullptr || sink == nullptr || grid < 1 || grid > 65536 || units < 1 || bytes >= (uint64_t(1) << 32) ||
      static_cast<uint64_t>(grid) * 8u * static_cast<uint64_t>(units) * 2048u > bytes)
    return -1;
  constexpr int D = 4;
  const size_t lds = 8u * (D + 1) * 2048u;
  if (hipFuncSetAttribute(reinterpret_cast<const void*>(lds_stream_kernel<D>), hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(lds)) != hipSuccess)
    return -2;
  hipLaunchKernelGGL(lds_stream_kernel<D>, dim3(grid), dim3(512), lds, stream, static_cast<const uint8_t*>(buf),
                     static_cast<uint32_t>(bytes), units, key, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}

// Read-stream probe: the measured HBM read rate that the decode GEMV is
// compared with.  Every 16-byte piece of a buffer is read once per launch by
// non-temporal 16-byte loads in a grid-stride loop, U pieces in flight per
// thread, and XOR-reduced per thread.  A thread stores its reduction only if
// it equals `key`, which the caller picks so that it never does for the data
// it fills in; the loads cannot be removed and nothing is written.
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

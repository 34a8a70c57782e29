// HBM read ceiling for the measurement of the decode kernels.
//
// Decode is bandwidth-bound: it moves every visible K/V byte once per step
// ("Multi-query attention", "Why this is a bandwidth argument, not a FLOP
// argument").  Its achieved GB/s is reported against the vendor's 8 TB/s and
// against what a plain read-only stream reaches on the same GPU in the same
// run.  This kernel is that stream: every byte of a buffer read once with
// the 128-bit non-temporal loads the decode kernels use, nothing written
// except, in the practically impossible case that the XOR of all words a
// thread read equals a fixed pattern, one word -- which keeps the loads live
// without adding traffic.
#include "gqa_device.h"
#include "gqa_launch.h"

namespace gqa {

constexpr int kReadThreads = 512;
constexpr int kReadUnroll = 8;  // 16-byte loads in flight per thread

// One workgroup per compute unit, each reading its own contiguous 1/W of the
// buffer, 64 KiB per step (the layout the decode kernels' key ranges give
// their workgroups).  Measured on MI355X with a 2 GiB buffer, this pattern
// reads ~7.1 TB/s against ~5.9 TB/s for a grid-stride loop over the whole
// buffer with the same loads.
__global__ __launch_bounds__(kReadThreads) void gqa_stream_read_kernel(const u32x4* __restrict__ p, long long n16,
                                                                       uint32_t* sink) {
  const long long per = (n16 + gridDim.x - 1) / gridDim.x;
  const long long lo = (long long)blockIdx.x * per;
  const long long hi = lo + per < n16 ? lo + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  long long i = lo + threadIdx.x;
  for (; i + (kReadUnroll - 1) * kReadThreads < hi; i += kReadUnroll * kReadThreads) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) v[u] = load_nt(p + i + u * kReadThreads);
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
  }
  for (; i < hi; i += kReadThreads) acc ^= load_nt(p + i);
  const uint32_t x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x9E3779B9u) *sink = x;
}

hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, int n_cu, hipStream_t stream) {
  const long long n16 = (long long)(bytes / 16);
  const dim3 grid(n_cu), block(kReadThreads);
  hipLaunchKernelGGL(gqa_stream_read_kernel, grid, block, 0, stream, static_cast<const u32x4*>(buf), n16, sink);
  return hipGetLastError();
}

}  // namespace gqa

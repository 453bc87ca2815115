// Streaming-read probe: the practical HBM read ceiling the attention kernels
// are compared against.  Each workgroup streams one contiguous part of the
// buffer with 16 independent 16-byte loads per thread per step and folds the
// data into one word per thread, so no load can be dropped.
#include "wmtp_device.hpp"
#include "wmtp_launch.hpp"

namespace wmtp {

constexpr int kStreamUnroll = 16;

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t nvec, int64_t per_wg,
                                                          uint32_t* __restrict__ sink) {
  const int64_t base = (int64_t)blockIdx.x * per_wg;
  const int64_t end = min(base + per_wg, nvec);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = base + threadIdx.x; i < end; i += 256 * kStreamUnroll) {
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      const int64_t j = i + (int64_t)u * 256;
      v[u] = j < end ? src[j] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) acc ^= v[u];
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t st) {
  const int64_t nvec = bytes / 16;
  const int64_t per_wg = (nvec + workgroups - 1) / workgroups;
  stream_read_kernel<<<workgroups, 256, 0, st>>>(static_cast<const u32x4*>(src), nvec, per_wg, sink);
  return hipGetLastError();
}

}  // namespace wmtp

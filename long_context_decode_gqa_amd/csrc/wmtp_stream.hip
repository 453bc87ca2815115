// Streaming-read probe: the practical HBM read ceiling the attention kernels
// are compared against.  Each workgroup streams one contiguous part of the
// buffer; every thread keeps two stages of kStreamUnroll non-temporal 16-byte
// loads in flight (the next stage is issued before the current one is
// consumed) and folds the data into one word, so no load can be dropped.  Loads past the
// part's end are clamped to its last element and not folded, so every load
// stays in bounds and every stage issues the same loads.
#include "wmtp_device.hpp"
#include "wmtp_launch.hpp"

namespace wmtp {

constexpr int kStreamUnroll = 4;
constexpr int kStreamThreads = 256;

__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t nvec,
                                                                     int64_t per_wg, uint32_t* __restrict__ sink) {
  constexpr int64_t kStep = (int64_t)kStreamThreads * kStreamUnroll;
  const int64_t base = (int64_t)blockIdx.x * per_wg;
  const int64_t end = min(base + per_wg, nvec);
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (base < end) {
    const int64_t nsteps = (end - base + kStep - 1) / kStep;
    u32x4 r[2][kStreamUnroll];
    auto issue = [&](int64_t s, int slot) {
      const int64_t s0 = base + min(s, nsteps - 1) * kStep + threadIdx.x;
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u)
        r[slot][u] = __builtin_nontemporal_load(src + min(s0 + (int64_t)u * kStreamThreads, end - 1));
    };
    auto consume = [&](int64_t s, int slot) {
      const int64_t s0 = base + s * kStep + threadIdx.x;
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u)
        if (s0 + (int64_t)u * kStreamThreads < end) acc ^= r[slot][u];
    };
    issue(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    int64_t s = 0;
    for (; s + 2 <= nsteps; s += 2) {
      issue(s + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      consume(s, 0);
      issue(s + 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      consume(s + 1, 1);
    }
    if (s < nsteps) consume(s, 0);
  }
  sink[(int64_t)blockIdx.x * kStreamThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t st) {
  const int64_t nvec = bytes / 16;
  const int64_t per_wg = (nvec + workgroups - 1) / workgroups;
  stream_read_kernel<<<workgroups, kStreamThreads, 0, st>>>(static_cast<const u32x4*>(src), nvec, per_wg, sink);
  return hipGetLastError();
}

}  // namespace wmtp

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

// Paged variant: two pools (K and V) read as runs of 2^run_shift bytes, in the
// order of a run list (run r = runs[r], clamped to the pool).  Workgroup w reads
// runs [w per, (w + 1) per) of both pools, two pipeline stages of kStreamUnroll
// non-temporal 16-byte loads per thread and pool; indices past its last vector
// are clamped.  This is the attention kernels' access pattern without their
// arithmetic: the practical ceiling for reading a paged cache in table order.
__global__ __launch_bounds__(kStreamThreads) void stream_read_paged_kernel(
    const u32x4* __restrict__ k, const u32x4* __restrict__ v, const int32_t* __restrict__ runs, int32_t nruns,
    int64_t pool_runs, int run_shift, int per, uint32_t* __restrict__ sink) {
  constexpr int kStep = kStreamThreads * kStreamUnroll;
  const int vec_shift = run_shift - 4;                        // 16-byte vectors per run = 2^vec_shift
  const int r0 = blockIdx.x * per;
  const int r1 = min(r0 + per, nruns);
  u32x4 acc = {0u, 0u, 0u, 0u};
  if (r0 < r1) {
    const int64_t total = (int64_t)(r1 - r0) << vec_shift;
    const int64_t nsteps = (total + kStep - 1) / kStep;
    const int64_t vmask = (1ll << vec_shift) - 1;
    u32x4 rk[2][kStreamUnroll], rv[2][kStreamUnroll];
    // A load group (256 threads x 16 bytes) is 4 KiB-aligned inside the
    // workgroup's vectors and a run holds a whole number of groups, so the run
    // id is uniform per group: a scalar load, which leaves the vector loads'
    // wait counts alone.
    const const_i32_ptr runs_c = as_const_i32(runs);
    auto issue = [&](int64_t st, int slot) {
      const int64_t g0 = min(st, nsteps - 1) * kStep;
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u) {
        const int64_t gj = min(g0 + (int64_t)u * kStreamThreads, total - 1);
        const int64_t j = min(gj + threadIdx.x, total - 1);
        int64_t run = runs_c[r0 + (int)(gj >> vec_shift)];
        run = run < 0 ? 0 : (run >= pool_runs ? pool_runs - 1 : run);
        const int64_t at = (run << vec_shift) + (j & vmask);
        rk[slot][u] = __builtin_nontemporal_load(k + at);
        rv[slot][u] = __builtin_nontemporal_load(v + at);
      }
    };
    auto consume = [&](int64_t st, int slot) {
      const int64_t s0 = st * kStep + threadIdx.x;
#pragma unroll
      for (int u = 0; u < kStreamUnroll; ++u)
        if (s0 + (int64_t)u * kStreamThreads < total) acc ^= rk[slot][u] ^ rv[slot][u];
    };
    issue(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    int64_t st = 0;
    for (; st + 2 <= nsteps; st += 2) {
      issue(st + 1, 1);
      __builtin_amdgcn_sched_barrier(0);
      consume(st, 0);
      issue(st + 2, 0);
      __builtin_amdgcn_sched_barrier(0);
      consume(st + 1, 1);
    }
    if (st < nsteps) consume(st, 0);
  }
  sink[(int64_t)blockIdx.x * kStreamThreads + threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

hipError_t launch_stream_read_paged(const void* k, const void* v, const int32_t* runs, int32_t nruns,
                                    int64_t pool_runs, int run_shift, uint32_t* sink, int workgroups,
                                    hipStream_t st) {
  const int per = (nruns + workgroups - 1) / workgroups;
  stream_read_paged_kernel<<<workgroups, kStreamThreads, 0, st>>>(static_cast<const u32x4*>(k),
                                                                  static_cast<const u32x4*>(v), runs, nruns,
                                                                  pool_runs, run_shift, per, sink);
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t st) {
  const int64_t nvec = bytes / 16;
  const int64_t per_wg = (nvec + workgroups - 1) / workgroups;
  stream_read_kernel<<<workgroups, kStreamThreads, 0, st>>>(static_cast<const u32x4*>(src), nvec, per_wg, sink);
  return hipGetLastError();
}

}  // namespace wmtp

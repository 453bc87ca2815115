// The matrix-core kernels at head_dim 64 and 128.  The one-row-tile kernel of
// wmtp_row_tile.hpp runs verify up to 32 packed rows and the draft step over the
// paged pool or the ring: each wave owns a 64-element slice of D, so a work
// item runs one wave (d = 64) or two (d = 128) and sums that many partial score
// tiles.  Verify of 33..96 rows runs on the two-team kernel of wmtp_teams.hpp:
// one loader wave per slice of D, and one compute wave per row tile over all of
// D.  These instantiations live in their own translation unit, apart from the
// head_dim 256 ones, whose instruction schedule is kept as measured.
#include "wmtp_launch.hpp"
#include "wmtp_row_tile.hpp"
#include "wmtp_teams.hpp"

namespace wmtp {

template <int D, int G>
static hipError_t launch_small_dg(bool single_query, bool ring, const SplitArgs& a, int grid, hipStream_t st) {
  constexpr int threads = D / kVQ * 64;
  constexpr int team_threads = (D / kVQ + 4) * 64;
  const int rows = single_query ? G : a.t_q * G;
  if (ring)
    mfma_attn_kernel<D, G, true, true><<<grid, threads, 0, st>>>(a);
  else if (single_query)
    mfma_attn_kernel<D, G, true, false><<<grid, threads, 0, st>>>(a);
  else if (rows <= 32)
    mfma_attn_kernel<D, G, false, false><<<grid, threads, 0, st>>>(a);
  else if (rows <= 64)
    mfma_attn_teams_kernel<D, G, 2><<<grid, team_threads, 0, st>>>(a);
  else
    mfma_attn_teams_kernel<D, G, 3><<<grid, team_threads, 0, st>>>(a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_small_d(int group, bool single_query, bool ring, const SplitArgs& a, int grid,
                                 hipStream_t st) {
  switch (group) {
    case 1: return launch_small_dg<D, 1>(single_query, ring, a, grid, st);
    case 2: return launch_small_dg<D, 2>(single_query, ring, a, grid, st);
    case 4: return launch_small_dg<D, 4>(single_query, ring, a, grid, st);
    case 8: return launch_small_dg<D, 8>(single_query, ring, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_row_tile_small(int head_dim, int group, bool single_query, bool ring, const SplitArgs& a, int grid,
                                 hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  const int rows = single_query ? group : a.t_q * group;
  if (rows > 3 * 32 || (ring && !single_query)) return hipErrorInvalidValue;
  switch (head_dim) {
    case 64: return launch_small_d<64>(group, single_query, ring, a, grid, st);
    case 128: return launch_small_d<128>(group, single_query, ring, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wmtp

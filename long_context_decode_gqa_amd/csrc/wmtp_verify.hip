// Verify launches on gfx950 matrix cores: the target's full-context attention
// of the gamma+1 drafted positions, and the native draft step (one query token
// over the whole paged cache).
//
// Up to 32 packed rows (one row tile) run on the one-row-tile kernel of
// wmtp_row_tile.hpp, instantiated here for the paged pool; 33..96 rows (two or
// three row tiles, gamma + 1 > 4 at G = 8) run on the two-team kernel below,
// which reads K and V the same way.
#include "wmtp_launch.hpp"
#include "wmtp_row_tile.hpp"
#include "wmtp_teams.hpp"

namespace wmtp {

template <int G>
static hipError_t launch_rt(int rt, bool single, const SplitArgs& a, int grid, hipStream_t st) {
  if (single) {
    mfma_attn_kernel<kVD, G, true, false><<<grid, 256, 0, st>>>(a);
  } else {
    switch (rt) {
      case 1: mfma_attn_kernel<kVD, G, false, false><<<grid, 256, 0, st>>>(a); break;
      case 2: mfma_attn_teams_kernel<kVD, G, 2><<<grid, 512, 0, st>>>(a); break;
      case 3: mfma_attn_teams_kernel<kVD, G, 3><<<grid, 512, 0, st>>>(a); break;
      default: return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

hipError_t launch_verify(int head_dim, int group, bool single_query, const SplitArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (head_dim != kVD) return hipErrorInvalidValue;
  const int rows = single_query ? group : a.t_q * group;
  const int rt = (rows + 31) / 32;
  switch (group) {
    case 1: return launch_rt<1>(rt, single_query, a, grid, st);
    case 2: return launch_rt<2>(rt, single_query, a, grid, st);
    case 4: return launch_rt<4>(rt, single_query, a, grid, st);
    case 8: return launch_rt<8>(rt, single_query, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wmtp

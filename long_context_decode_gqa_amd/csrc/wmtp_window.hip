// Window-mode draft step on gfx950 matrix cores: the one-row-tile kernel of
// wmtp_row_tile.hpp over the compact ring's visible entries (the sinks, then the
// window), for one query token with bf16 PV weights at head_dim 256.  Its work
// items are short (the window is split across the chip), so the kernel's
// register ring keeps a work item's tiles in flight together, and the score
// and PV contractions run on the matrix cores instead of the vector unit.
#include "wmtp_launch.hpp"
#include "wmtp_row_tile.hpp"

namespace wmtp {

template <int G>
static hipError_t launch_ring(const SplitArgs& a, int grid, hipStream_t st) {
  mfma_attn_kernel<kVD, G, true, true><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_window_mfma(int head_dim, int group, const SplitArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  if (head_dim != kVD) return hipErrorInvalidValue;
  switch (group) {
    case 1: return launch_ring<1>(a, grid, st);
    case 2: return launch_ring<2>(a, grid, st);
    case 4: return launch_ring<4>(a, grid, st);
    case 8: return launch_ring<8>(a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wmtp

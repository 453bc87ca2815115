// Host-side launchers of the Windowed-MTP kernels (internal to libwmtp).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "wmtp.h"
#include "wmtp_device.hpp"

namespace wmtp {

struct CombineArgs {
  const float* part_o;
  const float* part_lse;
  void* out;
  float* lse_out;
  int32_t rows;          // rows per sequence
  int32_t head_dim;
  int32_t batch;
  int32_t out_bf16;
  int32_t split_base[WMTP_MAX_BATCH + 1];
};

struct AppendArgs {
  const void* k_new;
  const void* v_new;
  void* k;
  void* v;
  const int32_t* block_table;   // paged
  int32_t* slot_pos;            // ring
  int64_t max_block;
  int32_t num_kv_heads;
  int32_t row_bytes;            // head_dim * element bytes
  int32_t run_rows;             // paged: token rows from one (block, head) run to the next
  int32_t t_new;
  int32_t bt_stride;
  int32_t sink;
  int32_t window;
  int32_t headroom;
  int32_t pos[WMTP_MAX_BATCH];  // first new position (appends) or kept length (rollback)
};

// The slice kernel (wmtp_draft.hip): window mode, and full mode with fp32 data, fp32 PV weights.
hipError_t launch_draft(int dtype, int head_dim, int group, bool window, const SplitArgs& a, int grid,
                        hipStream_t st);
// The native draft step in bf16 with fp32 softmax weights: each wave owns whole tiles of keys over
// all of head_dim (wmtp_draft_rows.hip).
hipError_t launch_draft_rows(int head_dim, int group, const SplitArgs& a, int grid, hipStream_t st);
// Matrix-core split-K attention over the paged pool (bf16, head_dim 256) for
// a.t_q query tokens, or for exactly one when single_query is set.
hipError_t launch_verify(int head_dim, int group, bool single_query, const SplitArgs& a, int grid, hipStream_t st);
// The same kernel for one query token over the ring's visible entries (window mode).
hipError_t launch_window_mfma(int head_dim, int group, const SplitArgs& a, int grid, hipStream_t st);
// The one-row-tile kernel at head_dim 64 or 128 (one or two waves per work item):
// verify of up to 32 packed rows, or a draft step over the paged pool or the ring.
hipError_t launch_row_tile_small(int head_dim, int group, bool single_query, bool ring, const SplitArgs& a, int grid,
                                 hipStream_t st);
hipError_t launch_combine(const CombineArgs& a, hipStream_t st);
hipError_t launch_ring_append(const AppendArgs& a, int batch, hipStream_t st);
hipError_t launch_paged_append(const AppendArgs& a, int batch, hipStream_t st);
hipError_t launch_ring_rollback(const AppendArgs& a, int batch, hipStream_t st);
hipError_t launch_debug_resolve_paged(const int32_t* bt_row, int32_t row_len, int64_t max_block, int num_kv_heads,
                                      int head_dim, int run_rows, int h, const int32_t* positions, int n,
                                      int64_t* out, hipStream_t st);
hipError_t launch_debug_resolve_ring(int sink, int cycle, const int32_t* positions, int n, int32_t* out,
                                     hipStream_t st);
hipError_t launch_debug_window_positions(int sink, int window, int headroom, int n, int32_t* out, hipStream_t st);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int workgroups, hipStream_t st);
hipError_t launch_stream_read_paged(const void* k, const void* v, const int32_t* runs, int32_t nruns,
                                    int64_t pool_runs, int run_shift, uint32_t* sink, int workgroups,
                                    hipStream_t st);

}  // namespace wmtp

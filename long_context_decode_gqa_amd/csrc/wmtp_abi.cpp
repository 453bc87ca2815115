// C ABI of libwmtp: argument checks, split planning and kernel dispatch.
//
// Every entry point validates all of its arguments before making any HIP call,
// so an invalid call enqueues nothing and can be tested on a machine without a
// GPU.  Nothing here allocates, synchronises or keeps state between calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>

#include <mutex>

#include "wmtp.h"
#include "wmtp_launch.hpp"

using namespace wmtp;

// Split partials of wmtp_draft_attn_noalloc, for callers that cannot allocate: one array per GPU
// that loads the library, held until the process ends.  Host code never names it except in the
// hipGetSymbolAddress call below; it uses the device address that call returns.
static __device__ __align__(256) uint8_t scratch[WMTP_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_dev_ptr[kMaxDevices] = {};

// Device address of the current device's scratch, resolved once per device with that device current.
int device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return WMTP_ELAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return WMTP_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_dev_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return WMTP_ELAUNCH;
    scratch_dev_ptr[dev] = p;
  }
  *out = scratch_dev_ptr[dev];
  return WMTP_OK;
}

}  // namespace

namespace {

constexpr int kDraftTile = 64;
constexpr int kVerifyTile = 32;    // keys per verify tile

// Default splits.  A split is one work item (sequence, KV head, split).  The
// default is the smallest split, a multiple of 64, whose work items fit one
// round of `slots` co-resident items (or of the smallest multiple of `slots`
// that holds one item per sequence and head), so no item waits for a second
// round.  Full-context launches target 256 slots, one item per MI355X compute
// unit: each CU streams one long run of blocks, measured faster than two
// co-resident items per CU at 1M keys (rows of 512 bytes or more; narrower
// rows target twice as many, see draft_plan).  Below about 32K keys the
// items are short and the launch is latency-bound: there the smallest split
// (64 entries) halves verify's launch at 2K keys against a floor of 256
// (8.1 against 14.4 us).  The window draft is latency-bound and its items fit
// two per CU (512-thread dot-product or 256-thread matrix-core items), so it
// targets 512 slots: longer items add a memory round trip of latency per 64
// entries.
constexpr int64_t kFullSlots = 256;
constexpr int64_t kWindowSlots = 512;
constexpr int64_t kFullMinSplit = 64;
constexpr int64_t kWindowMinSplit = 64;
constexpr int64_t kMaxDefaultSplit = 65536;

int64_t work_items(const int64_t* vis, int batch, int kv_heads, int64_t split) {
  int64_t n = 0;
  for (int b = 0; b < batch; ++b) n += (vis[b] + split - 1) / split;
  return n * kv_heads;
}

int32_t default_split(const int64_t* vis, int batch, int kv_heads, int64_t slots, int64_t min_split) {
  int64_t keys = 0;
  for (int b = 0; b < batch; ++b) keys += vis[b];
  int64_t target = slots;
  while (target < (int64_t)batch * kv_heads) target += slots;
  int64_t s = (keys * kv_heads + target - 1) / target;
  s = (s + kDraftTile - 1) / kDraftTile * kDraftTile;   // a multiple of both tiles
  s = s < min_split ? min_split : s;
  s = s > kMaxDefaultSplit ? kMaxDefaultSplit : s;
  while (s < kMaxDefaultSplit && work_items(vis, batch, kv_heads, s) > target) s += kDraftTile;
  return (int32_t)s;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elem_bytes(int dtype) { return dtype == WMTP_BF16 ? 2 : 4; }

int check_shape(const wmtp_shape* s) {
  if (!s) return WMTP_EINVAL;
  if (s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->num_q_heads % s->num_kv_heads != 0) return WMTP_EINVAL;
  if (s->dtype != WMTP_F32 && s->dtype != WMTP_BF16) return WMTP_EINVAL;
  if (!std::isfinite(s->scale)) return WMTP_EINVAL;
  const int g = s->num_q_heads / s->num_kv_heads;
  if (g != 1 && g != 2 && g != 4 && g != 8) return WMTP_EUNSUPPORTED;
  if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256) return WMTP_EUNSUPPORTED;
  return WMTP_OK;
}

int check_paged(const wmtp_paged* kv, bool need_table) {
  if (!kv || !kv->k || !kv->v) return WMTP_EINVAL;
  if (need_table && !kv->block_table) return WMTP_EINVAL;
  if (kv->block_size != WMTP_BLOCK_SIZE) return WMTP_EUNSUPPORTED;
  if (kv->max_blocks_per_seq <= 0 || kv->num_blocks <= 0) return WMTP_EINVAL;
  if (kv->run_rows != 0 && kv->run_rows < WMTP_BLOCK_SIZE) return WMTP_EINVAL;
  if (!aligned(kv->k, 16) || !aligned(kv->v, 16)) return WMTP_EALIGN;
  return WMTP_OK;
}

// Token rows from one (block, head) run to the next: 0 means 16 (separate pools).
int32_t run_rows_of(const wmtp_paged* kv) { return kv->run_rows ? kv->run_rows : WMTP_BLOCK_SIZE; }

int check_ring(const wmtp_ring* r) {
  if (!r || !r->k || !r->v || !r->slot_pos) return WMTP_EINVAL;
  if (r->sink < 0 || r->window < 1 || r->headroom < 0) return WMTP_EINVAL;
  if ((int64_t)r->sink + r->window + r->headroom > (int64_t)INT32_MAX / 2) return WMTP_EINVAL;
  if (!aligned(r->k, 16) || !aligned(r->v, 16) || !aligned(r->slot_pos, 4)) return WMTP_EALIGN;
  return WMTP_OK;
}

int64_t align256(int64_t x) { return (x + 255) & ~int64_t(255); }

struct Plan {
  int32_t total = 0;
  int32_t rows = 0;
  int32_t split_base[WMTP_MAX_BATCH + 1] = {};
  int64_t lse_off = 0;
  int64_t bytes = 0;
};

// Splits of `chunk` entries over per-sequence visible counts `vis`.
int make_plan(const int64_t* vis, int batch, int chunk, int rows, int head_dim, int kv_heads, Plan* p) {
  int64_t total = 0;
  p->split_base[0] = 0;
  for (int b = 0; b < batch; ++b) {
    total += (vis[b] + chunk - 1) / chunk;
    if (total * kv_heads > INT32_MAX) return WMTP_EINVAL;
    p->split_base[b + 1] = (int32_t)total;
  }
  p->total = (int32_t)total;
  p->rows = rows;
  const int64_t o_bytes = total * rows * (int64_t)head_dim * 4;
  p->lse_off = align256(o_bytes);
  p->bytes = p->lse_off + align256(total * rows * 4);
  return WMTP_OK;
}

// Window mode: the launch plans each sequence's visible count min(n, S_b + W_b)
// (S_b, W_b from the optional per-sequence arrays); the workspace size plans the
// bound min(n, S + W + R) that any policy stays under.  The default chunk comes
// from the bound in both, so a launch never needs more splits than the
// workspace size allowed for.
int draft_plan(int32_t mode, const wmtp_shape* shape, const int32_t* seq_lens, int32_t batch, int32_t chunk,
               int32_t sink, int32_t window, int32_t headroom, const int32_t* seq_sink, const int32_t* seq_window,
               bool upper_bound, Plan* p, int32_t* chunk_out) {
  int st = check_shape(shape);
  if (st) return st;
  const int base_mode = mode & 0xF;
  if (base_mode != WMTP_FULL && base_mode != WMTP_SINK_WINDOW) return WMTP_EINVAL;
  if ((mode & ~0xF) & ~WMTP_DRAFT_FAST_PV) return WMTP_EINVAL;
  if (!seq_lens || batch < 1 || batch > WMTP_MAX_BATCH) return WMTP_EINVAL;
  if (base_mode == WMTP_SINK_WINDOW &&
      (sink < 0 || window < 1 || headroom < 0 || (int64_t)sink + window + headroom > (int64_t)INT32_MAX / 2))
    return WMTP_EINVAL;
  const int64_t ring_slots = (int64_t)sink + window + headroom;
  int64_t vis[WMTP_MAX_BATCH], bound[WMTP_MAX_BATCH];
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < 0 || seq_lens[b] > WMTP_MAX_SEQ_LEN) return WMTP_EINVAL;
    if (base_mode == WMTP_FULL) {
      vis[b] = bound[b] = seq_lens[b];
      continue;
    }
    const int64_t sb = seq_sink ? seq_sink[b] : sink;
    const int64_t wb = seq_window ? seq_window[b] : window;
    if (sb < 0 || sb > sink || wb < 1 || wb > (int64_t)window + headroom) return WMTP_EINVAL;
    bound[b] = std::min<int64_t>(seq_lens[b], ring_slots);
    vis[b] = upper_bound ? bound[b] : std::min<int64_t>(seq_lens[b], sb + wb);
  }
  if (chunk == 0) {
    // Narrower rows mean fewer waves per work item (one per 64 bf16 elements on the
    // matrix-core kernel, 4 instead of 8 on the dot-product kernel below 512-byte
    // rows): target proportionally more items, so a CU holds as many waves' loads
    // (measured at 1M keys on the dot-product kernel: 4/1/64 137 -> 87 us, 8/1/128
    // 175 -> 130 us, 4/2/128 244 -> 194 us).  The count depends on the shape only,
    // so the workspace size does not depend on the PV flag.
    const int64_t row_bytes = (int64_t)shape->head_dim * elem_bytes(shape->dtype);
    const int64_t full_slots = kFullSlots * std::max<int64_t>(1, 512 / row_bytes);
    chunk = base_mode == WMTP_FULL ? default_split(bound, batch, shape->num_kv_heads, full_slots, kFullMinSplit)
                                   : default_split(bound, batch, shape->num_kv_heads, kWindowSlots, kWindowMinSplit);
  }
  if (chunk < kVerifyTile || chunk % kVerifyTile != 0) return WMTP_EINVAL;   // whole 32-key tiles
  *chunk_out = chunk;
  return make_plan(vis, batch, chunk, shape->num_q_heads, shape->head_dim, shape->num_kv_heads, p);
}

int verify_plan(const wmtp_shape* shape, int32_t t_q, const int32_t* seq_lens, int32_t batch, int32_t split,
                Plan* p, int32_t* split_out) {
  int st = check_shape(shape);
  if (st) return st;
  if (shape->dtype != WMTP_BF16) return WMTP_EUNSUPPORTED;
  if (!seq_lens || batch < 1 || batch > WMTP_MAX_BATCH) return WMTP_EINVAL;
  if (t_q < 1) return WMTP_EINVAL;
  const int g = shape->num_q_heads / shape->num_kv_heads;
  // up to three row tiles of 32 packed rows
  if ((int64_t)t_q * g > WMTP_MAX_VERIFY_ROWS) return WMTP_EUNSUPPORTED;
  int64_t vis[WMTP_MAX_BATCH];
  for (int b = 0; b < batch; ++b) {
    if (seq_lens[b] < t_q || seq_lens[b] > WMTP_MAX_SEQ_LEN) return WMTP_EINVAL;   // the queries' keys are cached
    vis[b] = seq_lens[b];
  }
  // A work item runs one wave per 64 elements of head_dim: narrower heads get
  // proportionally more items, so a CU still holds four waves' loads.
  if (split == 0)
    split = default_split(vis, batch, shape->num_kv_heads, kFullSlots * (256 / shape->head_dim), kFullMinSplit);
  if (split < kVerifyTile || split % kVerifyTile != 0) return WMTP_EINVAL;
  *split_out = split;
  return make_plan(vis, batch, split, t_q * shape->num_q_heads, shape->head_dim, shape->num_kv_heads, p);
}

void fill_parts(const Plan& p, void* ws, int batch, int head_dim, wmtp_partials* parts) {
  parts->o = static_cast<float*>(ws);
  parts->lse = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + p.lse_off);
  parts->batch = batch;
  parts->rows_per_seq = p.rows;
  parts->head_dim = head_dim;
  parts->total_splits = p.total;
  std::memset(parts->split_base, 0, sizeof(parts->split_base));
  for (int b = 0; b <= batch; ++b) parts->split_base[b] = p.split_base[b];
}

void fill_split_args(SplitArgs& a, const wmtp_shape* s, const Plan& p, const int32_t* seq_lens, int batch, int chunk,
                     const wmtp_partials* parts) {
  std::memset(&a, 0, sizeof(a));
  a.part_o = parts->o;
  a.part_lse = parts->lse;
  a.num_q_heads = s->num_q_heads;
  a.num_kv_heads = s->num_kv_heads;
  a.chunk = chunk;
  a.batch = batch;
  a.scale_log2 = s->scale * 1.44269504088896340736f;
  for (int b = 0; b <= batch; ++b) a.split_base[b] = p.split_base[b];
  for (int b = 0; b < batch; ++b) a.seq_len[b] = seq_lens[b];
}

int launch_status(hipError_t e) { return e == hipSuccess ? WMTP_OK : WMTP_ELAUNCH; }

// The output side of a combine: out (16-byte aligned), optional lse_out (4-byte aligned), dtype.
int check_combine_out(const void* out, const float* lse_out, int32_t out_dtype) {
  if (!out) return WMTP_EINVAL;
  if (out_dtype != WMTP_F32 && out_dtype != WMTP_BF16) return WMTP_EINVAL;
  if (!aligned(out, 16) || !aligned(lse_out, 4)) return WMTP_EALIGN;
  return WMTP_OK;
}

}  // namespace

extern "C" {

int64_t wmtp_draft_workspace_bytes(int32_t mode, const wmtp_shape* shape, const int32_t* seq_lens_host, int32_t batch,
                                   int32_t chunk_tokens, int32_t sink, int32_t window, int32_t headroom) {
  Plan p;
  int32_t chunk = 0;
  const int st = draft_plan(mode, shape, seq_lens_host, batch, chunk_tokens, sink, window, headroom, nullptr, nullptr,
                            true, &p, &chunk);
  return st ? st : p.bytes;
}

int64_t wmtp_verify_workspace_bytes(const wmtp_shape* shape, int32_t t_q, const int32_t* seq_lens_host, int32_t batch,
                                    int32_t split_tokens) {
  Plan p;
  int32_t split = 0;
  const int st = verify_plan(shape, t_q, seq_lens_host, batch, split_tokens, &p, &split);
  return st ? st : p.bytes;
}

}  // extern "C"

namespace {

// New tokens a fused call appends: none (t_new = 0), or t_new per sequence.
int check_new_tokens(const void* k_new, const void* v_new, int32_t t_new, const int32_t* seq_lens, int32_t batch) {
  if (t_new == 0) return WMTP_OK;
  if (!k_new || !v_new) return WMTP_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return WMTP_EALIGN;
  for (int b = 0; b < batch; ++b)
    if (seq_lens[b] < t_new) return WMTP_EINVAL;
  return WMTP_OK;
}

// check_only: run every argument check and the plan, then return before touching *parts or the GPU.
int draft_attn(int32_t mode, const wmtp_shape* shape, const void* q, const wmtp_paged* kv, const wmtp_ring* ring,
               const void* k_new, const void* v_new, int32_t t_new, const int32_t* seq_lens_host, int32_t batch,
               int32_t chunk_tokens, void* workspace, size_t workspace_bytes, wmtp_partials* parts, void* stream,
               bool check_only = false) {
  const int base_mode = mode & 0xF;
  int32_t sink = 0, window = 1, headroom = 0;
  if (base_mode == WMTP_SINK_WINDOW) {
    const int st = check_ring(ring);
    if (st) return st;
    sink = ring->sink;
    window = ring->window;
    headroom = ring->headroom;
  }
  Plan p;
  int32_t chunk = 0;
  const bool win = base_mode == WMTP_SINK_WINDOW;
  int st = draft_plan(mode, shape, seq_lens_host, batch, chunk_tokens, sink, window, headroom,
                      win ? ring->seq_sink : nullptr, win ? ring->seq_window : nullptr, false, &p, &chunk);
  if (st) return st;
  if (!q || !parts) return WMTP_EINVAL;
  if (!aligned(q, 16)) return WMTP_EALIGN;
  if (base_mode == WMTP_FULL) {
    st = check_paged(kv, true);
    if (st) return st;
    for (int b = 0; b < batch; ++b)
      if (((int64_t)seq_lens_host[b] + WMTP_BLOCK_SIZE - 1) / WMTP_BLOCK_SIZE > kv->max_blocks_per_seq)
        return WMTP_EINVAL;
  }
  if (base_mode == WMTP_SINK_WINDOW &&
      ((int64_t)ring->sink + ring->window + ring->headroom) * shape->head_dim * elem_bytes(shape->dtype) >
          (int64_t)INT32_MAX)
    return WMTP_EINVAL;   // lanes address the ring of one (sequence, head) with 32-bit offsets
  if (!workspace && p.bytes > 0) return WMTP_EINVAL;
  if (!aligned(workspace, 256)) return WMTP_EALIGN;
  if ((int64_t)workspace_bytes < p.bytes) return WMTP_EWORKSPACE;
  st = check_new_tokens(k_new, v_new, t_new, seq_lens_host, batch);
  if (st || check_only) return st;

  fill_parts(p, workspace, batch, shape->head_dim, parts);
  SplitArgs a;
  fill_split_args(a, shape, p, seq_lens_host, batch, chunk, parts);
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.t_new = t_new;
  if (base_mode == WMTP_FULL) {
    a.k = kv->k;
    a.v = kv->v;
    a.block_table = kv->block_table;
    a.bt_stride = kv->max_blocks_per_seq;
    a.max_block = kv->num_blocks - 1;
    a.run_rows = run_rows_of(kv);
  } else {
    a.k = ring->k;
    a.v = ring->v;
    a.slot_pos = ring->slot_pos;
    a.slots = ring->sink + ring->window + ring->headroom;
    a.sink = ring->sink;
    a.window = ring->window;
    for (int b = 0; b < batch; ++b) {
      a.seq_sink[b] = ring->seq_sink ? ring->seq_sink[b] : ring->sink;
      a.seq_window[b] = ring->seq_window ? ring->seq_window[b] : ring->window;
    }
  }
  const int grid = p.total * shape->num_kv_heads;
  const bool fast_pv = (mode & WMTP_DRAFT_FAST_PV) != 0 && shape->dtype == WMTP_BF16;
  if (fast_pv) {
    // A draft step is attention of a single query token, i.e. the verify
    // contraction with t_q = 1; both round p to bf16 before PV, so the G packed
    // rows run on the matrix-core kernel, which spends fewer vector instructions
    // per key than the vector kernels: over the paged context (native) or over
    // the ring's visible entries (window).
    a.t_q = 1;
    const int group = shape->num_q_heads / shape->num_kv_heads;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const bool window = base_mode == WMTP_SINK_WINDOW;
    if (shape->head_dim != 256)
      return launch_status(launch_row_tile_small(shape->head_dim, group, true, window, a, grid, st));
    return launch_status(window ? launch_window_mfma(shape->head_dim, group, a, grid, st)
                                : launch_verify(shape->head_dim, group, true, a, grid, st));
  }
  // The native step in bf16 with fp32 weights: whole tiles per wave, the scores summed and
  // exponentiated once per key and row (faster than the slice kernel at every head shape measured).
  if (shape->dtype == WMTP_BF16 && base_mode == WMTP_FULL)
    return launch_status(launch_draft_rows(shape->head_dim, shape->num_q_heads / shape->num_kv_heads, a, grid,
                                           static_cast<hipStream_t>(stream)));
  return launch_status(launch_draft(shape->dtype, shape->head_dim, shape->num_q_heads / shape->num_kv_heads,
                                    base_mode == WMTP_SINK_WINDOW, a, grid, static_cast<hipStream_t>(stream)));
}

int verify_attn(const wmtp_shape* shape, const void* q, int32_t t_q, const wmtp_paged* kv, const void* k_new,
                const void* v_new, int32_t t_new, const int32_t* seq_lens_host, int32_t batch, int32_t split_tokens,
                void* workspace, size_t workspace_bytes, wmtp_partials* parts, void* stream) {
  Plan p;
  int32_t split = 0;
  int st = verify_plan(shape, t_q, seq_lens_host, batch, split_tokens, &p, &split);
  if (st) return st;
  if (!q || !parts) return WMTP_EINVAL;
  if (!aligned(q, 16)) return WMTP_EALIGN;
  st = check_paged(kv, true);
  if (st) return st;
  for (int b = 0; b < batch; ++b)
    if (((int64_t)seq_lens_host[b] + WMTP_BLOCK_SIZE - 1) / WMTP_BLOCK_SIZE > kv->max_blocks_per_seq)
      return WMTP_EINVAL;
  if (!workspace && p.bytes > 0) return WMTP_EINVAL;
  if (!aligned(workspace, 256)) return WMTP_EALIGN;
  if ((int64_t)workspace_bytes < p.bytes) return WMTP_EWORKSPACE;
  st = check_new_tokens(k_new, v_new, t_new, seq_lens_host, batch);
  if (st) return st;

  fill_parts(p, workspace, batch, shape->head_dim, parts);
  SplitArgs a;
  fill_split_args(a, shape, p, seq_lens_host, batch, split, parts);
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.t_new = t_new;
  a.k = kv->k;
  a.v = kv->v;
  a.block_table = kv->block_table;
  a.bt_stride = kv->max_blocks_per_seq;
  a.max_block = kv->num_blocks - 1;
  a.run_rows = run_rows_of(kv);
  a.t_q = t_q;
  const int grid = p.total * shape->num_kv_heads;
  const int group = shape->num_q_heads / shape->num_kv_heads;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (shape->head_dim != 256)
    return launch_status(launch_row_tile_small(shape->head_dim, group, false, false, a, grid, hs));
  return launch_status(launch_verify(shape->head_dim, group, false, a, grid, hs));
}

}  // namespace

extern "C" {

int wmtp_draft_attn(int32_t mode, const wmtp_shape* shape, const void* q, const wmtp_paged* kv, const wmtp_ring* ring,
                    const int32_t* seq_lens_host, int32_t batch, int32_t chunk_tokens, void* workspace,
                    size_t workspace_bytes, wmtp_partials* parts, void* stream) {
  return draft_attn(mode, shape, q, kv, ring, nullptr, nullptr, 0, seq_lens_host, batch, chunk_tokens, workspace,
                    workspace_bytes, parts, stream);
}

int wmtp_draft_attn_append(int32_t mode, const wmtp_shape* shape, const void* q, const wmtp_paged* kv,
                           const wmtp_ring* ring, const void* k_new, const void* v_new, const int32_t* seq_lens_host,
                           int32_t batch, int32_t chunk_tokens, void* workspace, size_t workspace_bytes,
                           wmtp_partials* parts, void* stream) {
  if (!k_new || !v_new) return WMTP_EINVAL;
  return draft_attn(mode, shape, q, kv, ring, k_new, v_new, 1, seq_lens_host, batch, chunk_tokens, workspace,
                    workspace_bytes, parts, stream);
}

int wmtp_verify_attn(const wmtp_shape* shape, const void* q, int32_t t_q, const wmtp_paged* kv,
                     const int32_t* seq_lens_host, int32_t batch, int32_t split_tokens, void* workspace,
                     size_t workspace_bytes, wmtp_partials* parts, void* stream) {
  return verify_attn(shape, q, t_q, kv, nullptr, nullptr, 0, seq_lens_host, batch, split_tokens, workspace,
                     workspace_bytes, parts, stream);
}

int wmtp_verify_attn_append(const wmtp_shape* shape, const void* q, int32_t t_q, const wmtp_paged* kv,
                            const void* k_new, const void* v_new, const int32_t* seq_lens_host, int32_t batch,
                            int32_t split_tokens, void* workspace, size_t workspace_bytes, wmtp_partials* parts,
                            void* stream) {
  if (!k_new || !v_new) return WMTP_EINVAL;
  return verify_attn(shape, q, t_q, kv, k_new, v_new, t_q, seq_lens_host, batch, split_tokens, workspace,
                     workspace_bytes, parts, stream);
}

int wmtp_combine(const wmtp_partials* parts, void* out, float* lse_out, int32_t out_dtype, void* stream) {
  if (!parts) return WMTP_EINVAL;
  const int st = check_combine_out(out, lse_out, out_dtype);
  if (st) return st;
  if (out_dtype != WMTP_F32 && out_dtype != WMTP_BF16) return WMTP_EINVAL;
  if (parts->batch < 1 || parts->batch > WMTP_MAX_BATCH || parts->rows_per_seq < 1) return WMTP_EINVAL;
  if (parts->head_dim != 64 && parts->head_dim != 128 && parts->head_dim != 256) return WMTP_EUNSUPPORTED;
  if (parts->split_base[0] != 0 || parts->split_base[parts->batch] != parts->total_splits) return WMTP_EINVAL;
  for (int b = 0; b < parts->batch; ++b)
    if (parts->split_base[b + 1] < parts->split_base[b]) return WMTP_EINVAL;
  if (parts->total_splits > 0 && (!parts->o || !parts->lse)) return WMTP_EINVAL;
  if (!aligned(parts->o, 16)) return WMTP_EALIGN;
  CombineArgs a;
  std::memset(&a, 0, sizeof(a));
  a.part_o = parts->o;
  a.part_lse = parts->lse;
  a.out = out;
  a.lse_out = lse_out;
  a.rows = parts->rows_per_seq;
  a.head_dim = parts->head_dim;
  a.batch = parts->batch;
  a.out_bf16 = out_dtype == WMTP_BF16;
  for (int b = 0; b <= parts->batch; ++b) a.split_base[b] = parts->split_base[b];
  return launch_status(launch_combine(a, static_cast<hipStream_t>(stream)));
}

static int append_common(const wmtp_shape* shape, const void* k_new, const void* v_new, const int32_t* pos_host,
                         int32_t batch, int32_t t_new, AppendArgs* a) {
  int st = check_shape(shape);
  if (st) return st;
  if (!pos_host || batch < 1 || batch > WMTP_MAX_BATCH || t_new < 0) return WMTP_EINVAL;
  if (t_new > 0 && (!k_new || !v_new)) return WMTP_EINVAL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16)) return WMTP_EALIGN;
  if ((int64_t)batch * t_new > INT32_MAX) return WMTP_EINVAL;
  std::memset(a, 0, sizeof(*a));
  for (int b = 0; b < batch; ++b) {
    if (pos_host[b] < 0 || (int64_t)pos_host[b] + t_new > WMTP_MAX_SEQ_LEN) return WMTP_EINVAL;
    a->pos[b] = pos_host[b];
  }
  a->k_new = k_new;
  a->v_new = v_new;
  a->num_kv_heads = shape->num_kv_heads;
  a->row_bytes = shape->head_dim * elem_bytes(shape->dtype);
  a->t_new = t_new;
  return WMTP_OK;
}

int wmtp_ring_append(const wmtp_shape* shape, const wmtp_ring* ring, const void* k_new, const void* v_new,
                     const int32_t* pos_host, int32_t batch, int32_t t_new, void* stream) {
  int st = check_ring(ring);
  if (st) return st;
  AppendArgs a;
  st = append_common(shape, k_new, v_new, pos_host, batch, t_new, &a);
  if (st) return st;
  a.k = ring->k;
  a.v = ring->v;
  a.slot_pos = ring->slot_pos;
  a.sink = ring->sink;
  a.window = ring->window;
  a.headroom = ring->headroom;
  return launch_status(launch_ring_append(a, batch, static_cast<hipStream_t>(stream)));
}

int wmtp_ring_rollback(const wmtp_ring* ring, const int32_t* seq_lens_host, int32_t batch, void* stream) {
  int st = check_ring(ring);
  if (st) return st;
  if (!seq_lens_host || batch < 1 || batch > WMTP_MAX_BATCH) return WMTP_EINVAL;
  AppendArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int b = 0; b < batch; ++b) {
    if (seq_lens_host[b] < 0 || seq_lens_host[b] > WMTP_MAX_SEQ_LEN) return WMTP_EINVAL;
    a.pos[b] = seq_lens_host[b];
  }
  a.slot_pos = ring->slot_pos;
  a.sink = ring->sink;
  a.window = ring->window;
  a.headroom = ring->headroom;
  return launch_status(launch_ring_rollback(a, batch, static_cast<hipStream_t>(stream)));
}

int wmtp_paged_append(const wmtp_shape* shape, const wmtp_paged* kv, const void* k_new, const void* v_new,
                      const int32_t* pos_host, int32_t batch, int32_t t_new, void* stream) {
  int st = check_paged(kv, true);
  if (st) return st;
  AppendArgs a;
  st = append_common(shape, k_new, v_new, pos_host, batch, t_new, &a);
  if (st) return st;
  for (int b = 0; b < batch; ++b)
    if (((int64_t)pos_host[b] + t_new + WMTP_BLOCK_SIZE - 1) / WMTP_BLOCK_SIZE > kv->max_blocks_per_seq)
      return WMTP_EINVAL;
  a.k = kv->k;
  a.v = kv->v;
  a.block_table = kv->block_table;
  a.bt_stride = kv->max_blocks_per_seq;
  a.max_block = kv->num_blocks - 1;
  a.run_rows = run_rows_of(kv);
  return launch_status(launch_paged_append(a, batch, static_cast<hipStream_t>(stream)));
}

int wmtp_debug_resolve_paged(const wmtp_paged* kv, int32_t num_kv_heads, int32_t head_dim, int32_t b, int32_t h,
                             const int32_t* positions, int32_t n, int64_t* offsets_out, void* stream) {
  if (!kv || !kv->block_table || kv->block_size != WMTP_BLOCK_SIZE || kv->num_blocks <= 0) return WMTP_EINVAL;
  if (kv->max_blocks_per_seq <= 0 || num_kv_heads <= 0 || head_dim <= 0 || b < 0 || h < 0 || h >= num_kv_heads)
    return WMTP_EINVAL;
  if (kv->run_rows != 0 && kv->run_rows < WMTP_BLOCK_SIZE) return WMTP_EINVAL;
  if (n < 0 || (n > 0 && (!positions || !offsets_out))) return WMTP_EINVAL;
  if (!aligned(offsets_out, 8)) return WMTP_EALIGN;
  const int32_t* row = kv->block_table + (int64_t)b * kv->max_blocks_per_seq;
  return launch_status(launch_debug_resolve_paged(row, kv->max_blocks_per_seq, kv->num_blocks - 1, num_kv_heads,
                                                  head_dim, run_rows_of(kv), h, positions, n, offsets_out,
                                                  static_cast<hipStream_t>(stream)));
}

int wmtp_debug_resolve_ring(int32_t sink, int32_t window, int32_t headroom, const int32_t* positions, int32_t n,
                            int32_t* slots_out, void* stream) {
  if (sink < 0 || window < 1 || headroom < 0 || n < 0 || (n > 0 && (!positions || !slots_out))) return WMTP_EINVAL;
  if ((int64_t)sink + window + headroom > INT32_MAX / 2) return WMTP_EINVAL;
  return launch_status(launch_debug_resolve_ring(sink, window + headroom, positions, n, slots_out,
                                                 static_cast<hipStream_t>(stream)));
}

int wmtp_debug_window_positions(int32_t sink, int32_t window, int32_t headroom, int32_t n, int32_t* out,
                                void* stream) {
  if (sink < 0 || window < 1 || headroom < 0 || n < 0 || !out) return WMTP_EINVAL;
  if ((int64_t)sink + window + headroom > INT32_MAX / 2) return WMTP_EINVAL;
  return launch_status(
      launch_debug_window_positions(sink, window, headroom, n, out, static_cast<hipStream_t>(stream)));
}

int wmtp_plan_memory(const wmtp_shape* shape, int32_t target_layers, int64_t context, int32_t sink,
                     int32_t window, int32_t headroom, int64_t budget_bytes, wmtp_memory_plan* out) {
  const int st = check_shape(shape);
  if (st) return st;
  if (!out || target_layers < 0 || context < 1 || budget_bytes < 0) return WMTP_EINVAL;
  if (sink < 0 || window < 1 || headroom < 0 || (int64_t)sink + window + headroom > (int64_t)INT32_MAX / 2)
    return WMTP_EINVAL;
  const int64_t row = (int64_t)shape->num_kv_heads * shape->head_dim * elem_bytes(shape->dtype) * 2;   // K+V
  const int64_t blocks = (context + WMTP_BLOCK_SIZE - 1) / WMTP_BLOCK_SIZE;
  if (blocks > INT64_MAX / (WMTP_BLOCK_SIZE * row) / (target_layers + 1)) return WMTP_EINVAL;
  const int64_t layer = blocks * WMTP_BLOCK_SIZE * row;
  const int64_t table = blocks * 4;
  const int64_t ring = ((int64_t)sink + window + headroom) * (row + 4);
  out->layer_bytes = layer;
  out->block_table_bytes = table;
  out->ring_bytes = ring;
  out->native_seq_bytes = (int64_t)target_layers * layer + layer + table;
  out->windowed_seq_bytes = (int64_t)target_layers * layer + ring + table;
  // context >= 1 gives native_seq_bytes >= one block of K and V, and the ring at least one slot
  out->reclaimed_fraction = 1.0 - (double)out->windowed_seq_bytes / (double)out->native_seq_bytes;
  out->native_sequences = budget_bytes / out->native_seq_bytes;
  out->windowed_sequences = budget_bytes / out->windowed_seq_bytes;
  return WMTP_OK;
}

int wmtp_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (!src || !sink || bytes < 16 || workgroups < 1 || workgroups > (1 << 20)) return WMTP_EINVAL;
  if (!aligned(src, 16) || !aligned(sink, 4) || bytes % 16 != 0) return WMTP_EALIGN;
  return launch_status(launch_stream_read(src, bytes, sink, workgroups, static_cast<hipStream_t>(stream)));
}

int wmtp_stream_read_paged(const void* k, const void* v, int64_t pool_bytes, const int32_t* runs, int32_t nruns,
                           int32_t run_bytes, uint32_t* sink, int32_t workgroups, void* stream) {
  if (!k || !v || !runs || !sink || nruns < 1 || workgroups < 1 || workgroups > (1 << 20)) return WMTP_EINVAL;
  if (run_bytes < 4096 || run_bytes > (1 << 20) || (run_bytes & (run_bytes - 1)) != 0) return WMTP_EINVAL;
  if (pool_bytes < run_bytes) return WMTP_EINVAL;
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(runs, 4) || !aligned(sink, 4)) return WMTP_EALIGN;
  const int run_shift = __builtin_ctz((unsigned)run_bytes);
  return launch_status(launch_stream_read_paged(k, v, runs, nruns, pool_bytes / run_bytes, run_shift, sink, workgroups,
                                                static_cast<hipStream_t>(stream)));
}

int wmtp_draft_attn_noalloc(int32_t mode, const wmtp_shape* shape, const void* q, const wmtp_paged* kv,
                            const wmtp_ring* ring, const void* k_new, const void* v_new,
                            const int32_t* seq_lens_host, int32_t batch, int32_t chunk_tokens, void* out,
                            float* lse_out, int32_t out_dtype, void* stream) {
  if ((k_new == nullptr) != (v_new == nullptr)) return WMTP_EINVAL;
  const int32_t t_new = k_new ? 1 : 0;
  // Every check, including the plan's size against the fixed scratch, before any HIP call.
  wmtp_partials parts;
  int st = draft_attn(mode, shape, q, kv, ring, k_new, v_new, t_new, seq_lens_host, batch, chunk_tokens,
                      reinterpret_cast<void*>(uintptr_t{256}), WMTP_NOALLOC_SCRATCH_BYTES, &parts, stream, true);
  if (st) return st;
  st = check_combine_out(out, lse_out, out_dtype);
  if (st) return st;
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st) return st;
  st = draft_attn(mode, shape, q, kv, ring, k_new, v_new, t_new, seq_lens_host, batch, chunk_tokens, ws,
                  WMTP_NOALLOC_SCRATCH_BYTES, &parts, stream);
  if (st) return st;
  return wmtp_combine(&parts, out, lse_out, out_dtype, stream);
}

const char* wmtp_status_str(int status) {
  switch (status) {
    case WMTP_OK: return "ok";
    case WMTP_EINVAL: return "invalid argument";
    case WMTP_EUNSUPPORTED: return "unsupported shape or dtype";
    case WMTP_EALIGN: return "pointer not aligned";
    case WMTP_EWORKSPACE: return "workspace too small (or the plan exceeds the fixed scratch of the no-allocation call)";
    case WMTP_ELAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* wmtp_version(void) { return "wmtp 0.1 gfx950"; }

}  // extern "C"

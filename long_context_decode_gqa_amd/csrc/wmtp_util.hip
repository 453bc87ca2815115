// LSE combine, ring / paged append and index-resolution kernels for gfx950.
#include "wmtp_device.hpp"
#include "wmtp_launch.hpp"

namespace wmtp {

// ----------------------------------------------------------------------------- combine
// Flash-decoding merge of split partials.  A split holding the keys K_i gives
// (o_i, lse_i); the result over the union is
//   L = log sum_i exp(lse_i),  o = sum_i exp(lse_i - L) o_i.
// Workgroup = (sequence b, row r, 32-float slice of D: one 128-byte line per
// split).  Its NW waves are 8 lanes across the slice (16 bytes each) x 8 NW
// split lanes.  Every thread merges its own splits (all loads independent),
// then the 8 split lanes of a wave are merged with a shuffle tree and the NW
// waves through LDS.  A thread merges up to PER (4 or 8) splits per round of
// loads, and NW grows with the splits of the longest sequence, so up to 1,024
// splits take one round: with a fixed 4 waves the 1,024 splits of a
// one-KV-head draft at head_dim 64 over 1M keys gave each thread 32 splits.
constexpr int kCombineDL = 8;                     // lanes across a D slice (128 bytes)

struct MergeState {
  float m, w;
  f32x4 acc;
};

// Merge (m, w, acc) states that describe disjoint key sets (log2 domain).
__device__ __forceinline__ MergeState merge_state(const MergeState& x, const MergeState& y) {
  const float m = fmaxf(x.m, y.m);
  if (m == kNegInf) return x;
  const float fx = exp2f(x.m - m), fy = exp2f(y.m - m);
  return {m, x.w * fx + y.w * fy, x.acc * fx + y.acc * fy};
}

template <int NW, int PER>
__global__ __launch_bounds__(NW * 64) void combine_kernel(const CombineArgs a) {
  constexpr int SL = NW * 64 / kCombineDL;        // split lanes
  __shared__ MergeState sm[NW][kCombineDL];
  const int slices = a.head_dim / (4 * kCombineDL);
  const int slice = blockIdx.x % slices;
  const int br = blockIdx.x / slices;             // b * rows + r
  const int b = br / a.rows;
  const int r = br % a.rows;
  const int dl = threadIdx.x % kCombineDL;
  const int sl = threadIdx.x / kCombineDL;
  const int s0 = a.split_base[b], s1 = a.split_base[b + 1];
  const int d0 = slice * 4 * kCombineDL + dl * 4;

  // One pass over this thread's splits, merging each (lse, o) into a running
  // (m, w, acc) in log2 units.  The loads of up to PER splits
  // are issued before any of them is used: indexes past the sequence's last
  // split are clamped to its first and weighted out, and the merge has no
  // branch, so the loads of a round are in flight together (a branch per split
  // made each split one memory round trip of its own).  An empty split carries
  // lse = -inf and o = 0 and gets weight 0.
  MergeState st;
  st.m = kNegInf;
  st.w = 0.f;
  st.acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int base = s0 + sl; base < s1; base += PER * SL) {
    float l[PER];
    f32x4 x[PER];
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const int s = base + k * SL;
      const int sc = s < s1 ? s : s0;
      const float ls = a.part_lse[(int64_t)sc * a.rows + r];
      l[k] = s < s1 ? ls * kLog2e : kNegInf;
      x[k] = *reinterpret_cast<const f32x4*>(a.part_o + ((int64_t)sc * a.rows + r) * a.head_dim + d0);
    }
#pragma unroll
    for (int k = 0; k < PER; ++k) {
      const float mn = fmaxf(st.m, l[k]);
      const float ref = mn == kNegInf ? 0.f : mn;       // both -inf: fa = fb = 0
      const float fa = exp2f(st.m - ref), fb = exp2f(l[k] - ref);
      st.acc = st.acc * fa + fb * x[k];
      st.w = st.w * fa + fb;
      st.m = mn;
    }
  }
  // merge tree over the split lanes of this wave (lane = kCombineDL sl + dl):
  // partners 8, 16 and 32 lanes away, exchanged without LDS
  auto merge_with = [&](auto partner) {
    MergeState o;
    o.m = partner(st.m);
    o.w = partner(st.w);
#pragma unroll
    for (int e = 0; e < 4; ++e) o.acc[e] = partner(st.acc[e]);
    st = merge_state(st, o);
  };
  static_assert(kCombineDL == 8, "the merge tree starts 8 lanes apart");
  merge_with([](float x) { return lane_xor<8>(x); });
  merge_with([](float x) { return lane_xor<16>(x); });
  merge_with([](float x) { return lane_xor<32>(x); });
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) < kCombineDL) sm[wave][dl] = st;
  __syncthreads();
  if (threadIdx.x >= kCombineDL) return;
  MergeState t = sm[0][dl];
#pragma unroll
  for (int w = 1; w < NW; ++w) t = merge_state(t, sm[w][dl]);
  const float inv = t.w > 0.f ? 1.f / t.w : 0.f;
  const int64_t orow = ((int64_t)b * a.rows + r) * a.head_dim + d0;
  if (a.out_bf16) {
    uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<__bf16*>(a.out) + orow);
    o[0] = pack_bf16x2(t.acc[0] * inv, t.acc[1] * inv);
    o[1] = pack_bf16x2(t.acc[2] * inv, t.acc[3] * inv);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + orow) = t.acc * inv;
  }
  if (a.lse_out && slice == 0 && dl == 0)
    a.lse_out[(int64_t)b * a.rows + r] = t.w > 0.f ? (t.m + __log2f(t.w)) * kLn2 : kNegInf;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t st) {
  const int slices = a.head_dim / (4 * kCombineDL);
  const int grid = a.batch * a.rows * slices;
  if (grid <= 0) return hipSuccess;
  int most = 0;
  for (int b = 0; b < a.batch; ++b) most = std::max(most, a.split_base[b + 1] - a.split_base[b]);
  constexpr int L = 64 / kCombineDL;   // split lanes per wave
  if (most <= 4 * L * 4)
    combine_kernel<4, 4><<<grid, 4 * 64, 0, st>>>(a);
  else if (most <= 4 * L * 8)
    combine_kernel<4, 8><<<grid, 4 * 64, 0, st>>>(a);
  else if (most <= 8 * L * 8)
    combine_kernel<8, 8><<<grid, 8 * 64, 0, st>>>(a);
  else
    combine_kernel<16, 8><<<grid, 16 * 64, 0, st>>>(a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- appends
// One workgroup per (sequence, new token); threads copy 16-byte pieces of the
// token's H_kv rows of K and V.
__global__ __launch_bounds__(256) void ring_append_kernel(const AppendArgs a) {
  const int b = blockIdx.x / a.t_new;
  const int i = blockIdx.x % a.t_new;
  const int p = a.pos[b] + i;
  const int last = a.pos[b] + a.t_new - 1;
  const int cycle = a.window + a.headroom;
  if (!(p < a.sink || p > last - cycle)) return;          // overwritten later in this append
  const int slots = a.sink + cycle;
  const int slot = ring_slot(p, a.sink, cycle);
  const int pieces = a.row_bytes / 16;                     // per head
  const int64_t src_tok = ((int64_t)b * a.t_new + i) * a.num_kv_heads * a.row_bytes;
  for (int j = threadIdx.x; j < 2 * a.num_kv_heads * pieces; j += blockDim.x) {
    const int which = j / (a.num_kv_heads * pieces);       // 0 = K, 1 = V
    const int hp = j % (a.num_kv_heads * pieces);
    const int h = hp / pieces, pc = hp % pieces;
    const uint8_t* src = static_cast<const uint8_t*>(which ? a.v_new : a.k_new) + src_tok +
                         (int64_t)h * a.row_bytes + pc * 16;
    uint8_t* dst = static_cast<uint8_t*>(which ? a.v : a.k) +
                   (((int64_t)b * a.num_kv_heads + h) * slots + slot) * a.row_bytes + pc * 16;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
  if (threadIdx.x == 0) a.slot_pos[(int64_t)b * slots + slot] = p;
}

__global__ __launch_bounds__(256) void paged_append_kernel(const AppendArgs a) {
  const int b = blockIdx.x / a.t_new;
  const int i = blockIdx.x % a.t_new;
  const int64_t p = (int64_t)a.pos[b] + i;
  const int32_t* bt_row = a.block_table + (int64_t)b * a.bt_stride;
  const int64_t blk = paged_block_of(bt_row, p, a.max_block);
  const int pieces = a.row_bytes / 16;
  const int64_t src_tok = ((int64_t)b * a.t_new + i) * a.num_kv_heads * a.row_bytes;
  for (int j = threadIdx.x; j < 2 * a.num_kv_heads * pieces; j += blockDim.x) {
    const int which = j / (a.num_kv_heads * pieces);
    const int hp = j % (a.num_kv_heads * pieces);
    const int h = hp / pieces, pc = hp % pieces;
    const uint8_t* src = static_cast<const uint8_t*>(which ? a.v_new : a.k_new) + src_tok +
                         (int64_t)h * a.row_bytes + pc * 16;
    uint8_t* dst = static_cast<uint8_t*>(which ? a.v : a.k) +
                   paged_block_run(blk, h, a.num_kv_heads, (int64_t)a.run_rows * a.row_bytes) +
                   (p % kBlock) * a.row_bytes + pc * 16;
    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
  }
}

// Rollback: one workgroup per sequence clears the tag of every slot holding a
// position >= the kept length a.pos[b].
__global__ __launch_bounds__(256) void ring_rollback_kernel(const AppendArgs a) {
  const int b = blockIdx.x;
  const int slots = a.sink + a.window + a.headroom;
  int32_t* tags = a.slot_pos + (int64_t)b * slots;
  for (int s = threadIdx.x; s < slots; s += blockDim.x)
    if (tags[s] >= a.pos[b]) tags[s] = -1;
}

hipError_t launch_ring_rollback(const AppendArgs& a, int batch, hipStream_t st) {
  if (batch <= 0) return hipSuccess;
  ring_rollback_kernel<<<batch, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_ring_append(const AppendArgs& a, int batch, hipStream_t st) {
  const int grid = batch * a.t_new;
  if (grid <= 0) return hipSuccess;
  ring_append_kernel<<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_paged_append(const AppendArgs& a, int batch, hipStream_t st) {
  const int grid = batch * a.t_new;
  if (grid <= 0) return hipSuccess;
  paged_append_kernel<<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

// ----------------------------------------------------------------------------- index-resolution hooks
__global__ void debug_resolve_paged_kernel(const int32_t* bt_row, int32_t row_len, int64_t max_block,
                                           int num_kv_heads, int head_dim, int run_rows, int h,
                                           const int32_t* positions, int n, int64_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const int32_t p = positions[i];
  out[i] = (p < 0 || p / kBlock >= row_len)
               ? -1
               : paged_elem_offset(bt_row, p, h, num_kv_heads, head_dim, max_block, run_rows);
}

__global__ void debug_resolve_ring_kernel(int sink, int cycle, const int32_t* positions, int n, int32_t* out) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) out[i] = ring_slot(positions[i], sink, cycle);
}

// Slot -> visible position for a query at length n: slot s < S holds sink s;
// ring slot s holds the most recent p < n with slot(p) = s, if it is visible.
__global__ void debug_window_positions_kernel(int sink, int window, int cycle, int n, int32_t* out) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= sink + cycle) return;
  int32_t p;
  if (s < sink) {
    p = s < n ? s : -1;
  } else if (n <= sink) {
    p = -1;
  } else {
    const int32_t last = n - 1;                          // newest position, last >= sink
    const int32_t r = (last - sink) % cycle;             // its ring index
    const int32_t d = ((r - (s - sink)) % cycle + cycle) % cycle;
    p = last - d;                                        // newest position mapped to slot s
    if (p < sink || !window_visible(p, n, sink, window)) p = -1;
  }
  out[s] = p;
}

hipError_t launch_debug_resolve_paged(const int32_t* bt_row, int32_t row_len, int64_t max_block, int num_kv_heads,
                                      int head_dim, int run_rows, int h, const int32_t* positions, int n,
                                      int64_t* out, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  debug_resolve_paged_kernel<<<(n + 255) / 256, 256, 0, st>>>(bt_row, row_len, max_block, num_kv_heads, head_dim,
                                                             run_rows, h, positions, n, out);
  return hipGetLastError();
}

hipError_t launch_debug_resolve_ring(int sink, int cycle, const int32_t* positions, int n, int32_t* out,
                                     hipStream_t st) {
  if (n <= 0) return hipSuccess;
  debug_resolve_ring_kernel<<<(n + 255) / 256, 256, 0, st>>>(sink, cycle, positions, n, out);
  return hipGetLastError();
}

hipError_t launch_debug_window_positions(int sink, int window, int headroom, int n, int32_t* out, hipStream_t st) {
  const int slots = sink + window + headroom;
  if (slots <= 0) return hipSuccess;
  debug_window_positions_kernel<<<(slots + 255) / 256, 256, 0, st>>>(sink, window, window + headroom, n, out);
  return hipGetLastError();
}

}  // namespace wmtp

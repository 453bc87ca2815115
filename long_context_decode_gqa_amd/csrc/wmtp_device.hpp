// Device-side building blocks of the Windowed-MTP decode-attention kernels
// (gfx950 / CDNA4, wave64): kernel argument blocks, the paged and ring index
// resolvers, bf16 helpers and wave-level reductions.
//
// Index resolution follows the problem statement of "Windowed-MTP: Removing
// the Full-Context Draft-KV Tax at Million-Token Context" (arxivlens.com
// summary, Abstract): the native draft reads the whole paged cache, the
// windowed draft reads sink + window entries kept in a compact ring buffer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "wmtp.h"

namespace wmtp {

// ----------------------------------------------------------------------------- vector types
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kBlock = WMTP_BLOCK_SIZE;   // tokens per paged block

// Read-only data that every lane of a wave reads at the same address (the
// query rows) is read through the constant address space, which the compiler
// turns into scalar loads into SGPRs.  Only for buffers no kernel writes.
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;
__device__ __forceinline__ const_u32_ptr as_const_u32(const void* p) {
  return reinterpret_cast<const_u32_ptr>(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ const_i32_ptr as_const_i32(const void* p) {
  return reinterpret_cast<const_i32_ptr>(reinterpret_cast<uintptr_t>(p));
}

// Load from a wave-uniform 64-bit base plus a 32-bit per-lane byte offset, the
// form the global_load "saddr + voffset" addressing mode takes directly.
template <typename T>
__device__ __forceinline__ T load_at(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const T*>(base + off);
}

// Same, marked non-temporal (global_load ... nt): for K/V that one launch reads
// exactly once.  On MI355X a plain 2 GiB stream reads about 6.2 TB/s with
// ordinary loads and about 7.2 TB/s with non-temporal ones.
template <typename T>
__device__ __forceinline__ T load_nt(const uint8_t* base, uint32_t off) {
  if constexpr (std::is_same_v<T, uint2>) {   // HIP's struct vector: load the native 2-lane vector
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(base + off));
    return make_uint2(v[0], v[1]);
  } else {
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(base + off));
  }
}

// ----------------------------------------------------------------------------- kernel arguments
// Passed by value (kernarg segment); per-sequence lengths and split offsets ride
// along so that no host-to-device copy is needed before a launch.
struct SplitArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* block_table;   // paged source
  const int32_t* slot_pos;      // ring source
  float* part_o;
  float* part_lse;
  int64_t max_block;            // num_blocks - 1: block ids are clamped to this
  int32_t run_rows;             // paged: token rows from one (block, head) run to the next
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t bt_stride;            // max_blocks_per_seq
  int32_t slots;                // ring slots (sink + window + headroom)
  int32_t sink;
  int32_t window;
  int32_t chunk;                // entries per split
  int32_t batch;
  int32_t t_q;                  // verify: query tokens per sequence
  float scale_log2;             // scale * log2(e)
  int32_t split_base[WMTP_MAX_BATCH + 1];
  int32_t seq_len[WMTP_MAX_BATCH];
  int32_t seq_sink[WMTP_MAX_BATCH];      // ring: per-sequence sinks and window of the query
  int32_t seq_window[WMTP_MAX_BATCH];
  // Fused append: the step's t_new new tokens per sequence (positions n - t_new
  // .. n - 1), [batch][t_new][H_kv][D], written into k / v (and, for the ring,
  // their slot tags into slot_pos) before they are read.  t_new = 0: none.
  const void* k_new;
  const void* v_new;
  int32_t t_new;
};

// ----------------------------------------------------------------------------- resolvers
// Paged pool: (block, head) runs of 16 token rows, run_rows rows apart (16:
// separate K and V pools [block][kv_head][16][D]; 32: K and V of a run
// interleaved [block][kv_head][2][16][D]).  The byte offset of the start of a run.
__device__ __forceinline__ int64_t paged_block_run(int64_t blk, int h, int num_kv_heads, int64_t run_bytes) {
  return (blk * num_kv_heads + h) * run_bytes;
}

// Physical block of logical token t of a sequence (block-table row `bt_row`),
// clamped to the pool so a corrupt table cannot send a load out of bounds.
__device__ __forceinline__ int64_t clamp_block(int64_t blk, int64_t max_block) {
  blk = blk < 0 ? 0 : blk;
  return blk > max_block ? max_block : blk;
}
__device__ __forceinline__ int64_t paged_block_of(const int32_t* bt_row, int64_t t, int64_t max_block) {
  return clamp_block(bt_row[t / kBlock], max_block);
}
// Same, for a wave-uniform token: the table entry comes in through a scalar load.
__device__ __forceinline__ int64_t paged_block_uniform(const_i32_ptr bt_row, int64_t t, int64_t max_block) {
  return clamp_block(bt_row[t / kBlock], max_block);
}

// Element offset of (token t, head h, d = 0) in the paged pool.
__device__ __forceinline__ int64_t paged_elem_offset(const int32_t* bt_row, int64_t t, int h, int num_kv_heads,
                                                     int head_dim, int64_t max_block, int run_rows) {
  const int64_t blk = paged_block_of(bt_row, t, max_block);
  return ((blk * num_kv_heads + h) * run_rows + (t % kBlock)) * (int64_t)head_dim;
}

// Compact ring: sinks keep slots 0..S-1, later positions cycle through the
// `cycle` = W + R slots S..S+cycle-1 (R headroom slots absorb rejected drafts).
__device__ __forceinline__ int32_t ring_slot(int32_t p, int32_t sink, int32_t cycle) {
  return p < sink ? p : sink + (p - sink) % cycle;
}

// Is absolute position p in the sink + window visible set of a query at length n?
__device__ __forceinline__ bool window_visible(int32_t p, int32_t n, int32_t sink, int32_t window) {
  return p >= 0 && p < n && (p < sink || p >= n - window);
}

// Sequence owning global split `sg` (split_base is ascending; batch <= 64).
__device__ __forceinline__ int seq_of_split(const SplitArgs& a, int sg) {
  int b = 0;
  while (b + 1 < a.batch && a.split_base[b + 1] <= sg) ++b;
  return b;
}

// Window mode: the visible entries of sequence b's query at length n, in
// position order.  Entry t < s_vis is sink t; entry t >= s_vis is position
// w_start + t - s_vis, one of the last W_b positions before n.  slot(t) is the
// ring slot that holds it: positions below the layout's S keep their own slot,
// later ones cycle through the C = slots - S others.  The window spans at most
// C positions, so its cycle index wraps at most once from ws_mod, the cycle
// index of w_start: no per-lane division.
struct WindowView {
  int s_vis = 0, w_start = 0, nvis = 0, sink = 0, cycle = 1, ws_mod = 0;
  WindowView() = default;
  __device__ __forceinline__ WindowView(const SplitArgs& a, int b, int n) {
    s_vis = min(a.seq_sink[b], n);
    w_start = max(s_vis, n - a.seq_window[b]);
    nvis = s_vis + (n - w_start);
    sink = a.sink;
    cycle = a.slots - a.sink;
    ws_mod = (w_start >= sink && cycle > 0) ? (w_start - sink) % cycle : 0;
  }
  __device__ __forceinline__ int pos(int t) const { return t < s_vis ? t : w_start + (t - s_vis); }
  __device__ __forceinline__ int slot(int t) const {
    const int p = pos(t);
    if (p < sink) return p;
    const int c = w_start >= sink ? ws_mod + (p - w_start) : p - sink;
    return sink + (c >= cycle ? c - cycle : c);
  }
};

// Fused append: write the step's new tokens at positions [lo, hi) of sequence
// b, KV head h, into the cache (paged through the block table, or the ring
// with the slot tag), then make them visible to the whole workgroup before
// any of its loads.  Callers pass the positions that fall in the work item's
// own key range, so each (position, head) row has one writer and no other
// work item of the launch reads it; a ring tag is shared by the heads, and
// each head's writer stores the same value before reading it.  lo >= hi (no
// new token here) must hold for the whole workgroup or for none of it.
template <bool RING>
__device__ __forceinline__ void append_own_rows(const SplitArgs& a, int b, int h, int n, int lo, int hi,
                                                int row_bytes) {
  if (lo >= hi) return;
  const int Hkv = a.num_kv_heads;
  const int pieces = row_bytes / 16;
  const int cnt = hi - lo;
  const int first = n - a.t_new;                 // position of new token 0
  uint8_t* const k = static_cast<uint8_t*>(const_cast<void*>(a.k));
  uint8_t* const v = static_cast<uint8_t*>(const_cast<void*>(a.v));
  const int cycle = a.slots - a.sink;
  for (int j = threadIdx.x; j < 2 * cnt * pieces; j += blockDim.x) {
    const int which = j / (cnt * pieces);        // 0 = K, 1 = V
    const int r = j % (cnt * pieces);
    const int p = lo + r / pieces, pc = r % pieces;
    const int64_t src = (((int64_t)b * a.t_new + (p - first)) * Hkv + h) * row_bytes + pc * 16;
    int64_t dst;
    if constexpr (RING) {
      dst = (((int64_t)b * Hkv + h) * a.slots + ring_slot(p, a.sink, cycle)) * row_bytes;
    } else {
      const int64_t blk = paged_block_of(a.block_table + (int64_t)b * a.bt_stride, p, a.max_block);
      dst = paged_block_run(blk, h, Hkv, (int64_t)a.run_rows * row_bytes) + (int64_t)(p % kBlock) * row_bytes;
    }
    const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(which ? a.v_new : a.k_new) + src);
    *reinterpret_cast<u32x4*>((which ? v : k) + dst + pc * 16) = x;
  }
  if constexpr (RING) {
    int32_t* tags = const_cast<int32_t*>(a.slot_pos) + (int64_t)b * a.slots;
    for (int p = lo + (int)threadIdx.x; p < hi; p += blockDim.x) tags[ring_slot(p, a.sink, cycle)] = p;
  }
  __syncthreads();   // workgroup-scope release/acquire: the rows are visible to every wave's loads
}

// ----------------------------------------------------------------------------- numbers
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round to bf16 (RNE) and return the rounded value as fp32.
__device__ __forceinline__ float round_bf16(float x) {
  const __bf16 b = (__bf16)x;
  return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// Two fp32 values -> packed bf16x2 (RNE), `lo` in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));   // one v_cvt_pk_bf16_f32
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ----------------------------------------------------------------------------- wave reductions
// All cross-lane steps are VALU: DPP permutes inside 16-lane rows and gfx950's
// v_permlane16_swap / v_permlane32_swap across rows, so a reduction costs six
// dependent VALU operations and no LDS round trip.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]: lane ^ 1
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]: lane ^ 2
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i inside each 8 lanes
constexpr int kDppMirror = 0x140;       // lane i <-> 15 - i inside each 16-lane row
constexpr int kDppRowRor = 0x120;       // + s: rotate by s inside each 16-lane row

// value of the partner row (rows of 16 lanes paired 0-1, 2-3), combined
__device__ __forceinline__ float rows16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float rows16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max / sum of lane l and lane l ^ 32 (gfx950 v_permlane32_swap: a VALU swap
// of the two 32-lane halves, no LDS round trip).
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max / sum over all 64 lanes, returned in every lane (the sum's rounding
// order may differ between lanes)
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppMirror>(x));
  return halves_max(rows16_max(x));
}
__device__ __forceinline__ float wave_sum(float x) {
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  x += dpp_f32<kDppMirror>(x);
  return halves_sum(rows16_sum(x));
}

// The value of lane (this lane ^ M) for M = 8, 16, 32: a rotation by 8 inside
// the 16-lane row, or the row / half swaps (which hand each lane both its own
// and its partner's value; the lane's row parity picks the partner's).
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
  static_assert(M == 8 || M == 16 || M == 32, "partner distance 8, 16 or 32");
  const int lane = __lane_id();
  if constexpr (M == 8) {
    return dpp_f32<kDppRowRor + 8>(x);
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(((lane >> 4) & 1) ? r[0] : r[1]);
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(((lane >> 5) & 1) ? r[0] : r[1]);
  }
}

// Sum over the lanes congruent to this lane modulo STRIDE (a power of two):
// rotations by STRIDE, 2 STRIDE, ... inside the 16-lane rows, then the row swaps.
template <int STRIDE>
__device__ __forceinline__ float strided_lane_sum(float x) {
  static_assert(STRIDE >= 1 && STRIDE <= 64 && (STRIDE & (STRIDE - 1)) == 0, "power-of-two stride");
  if constexpr (STRIDE <= 1) x += dpp_f32<kDppXor1>(x);
  if constexpr (STRIDE <= 2) x += dpp_f32<kDppRowRor + 2>(x);
  if constexpr (STRIDE <= 4) x += dpp_f32<kDppRowRor + 4>(x);
  if constexpr (STRIDE <= 8) x += dpp_f32<kDppRowRor + 8>(x);
  if constexpr (STRIDE <= 16) x = rows16_sum(x);
  if constexpr (STRIDE <= 32) x = halves_sum(x);
  return x;
}

// 2^x on the hardware exponential (v_exp_f32): exp2(-inf) = 0; results below
// the fp32 normal range flush to zero, far below what a softmax weight of a
// kept row can contribute.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr uint32_t kBf16One2 = 0x3f803f80u;   // bf16 pair (1, 1)

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

}  // namespace wmtp

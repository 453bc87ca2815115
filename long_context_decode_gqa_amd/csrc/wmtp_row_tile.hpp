// Attention of a few query tokens over a long KV cache on gfx950 matrix cores,
// one row tile (up to 32 packed rows) per work item: the target's verify of the
// gamma+1 drafted positions, and the draft step (one query token) over the
// paged context (native) or over the compact ring (window).
//
// The target keeps full attention while it verifies the drafted positions
// ("Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
// Context", arxivlens summary, Abstract; howtospark case study, Method: one
// batched verify per cycle).  Per KV head the t_q query tokens x G query heads
// form packed rows, so QK^T and PV are real dense contractions (rows x
// head_dim against each key tile) and run on v_mfma_f32_32x32x16_bf16.  With
// t_q = 1 this is the MTP draft step: over the whole cache its read grows with
// the context; over the sinks and the window held in the ring it does not
// (same summary, Abstract).
//
// Work item = (sequence, KV head, split of `chunk` keys); one 256-thread
// workgroup whose 4 waves each own a quarter of head_dim.  Each wave keeps a
// 3-slot register ring of K/V tiles, so two tiles are in flight while a third
// is computed.  Per 32-key tile:
//   S^T = K Q^T     each wave contracts its quarter of D: A = its quarter of
//                   the K rows, moved from registers into a swizzled
//                   wave-private LDS stage and read back with lane = key,
//                   B = its quarter of Q^T held in registers.  The 4
//                   partial score tiles are summed through LDS (one barrier per
//                   tile), so every wave holds the full scores: lane l has
//                   packed row l % 32 for 16 keys.
//   softmax         row max over 16 registers and the partner half-wave
//                   (v_permlane32_swap); causal mask for query token i: key <=
//                   n - t_q + i, applied only on tiles that reach a boundary;
//                   lazy running maximum (rescale only on a 2^8 jump); the
//                   score scale folds into the exponent, p = 2^(s c - M).
//                   Identical in all waves, so the waves share one state.
//   O += P V        A = P straight from the score accumulator (bf16); B = V of
//                   the wave's quarter of D, 2 values per lane and key,
//                   regrouped into key pairs with v_perm_b32.
// The split writes o and lse for every packed row; the LSE combine merges
// splits.
//
// The template is instantiated in two translation units: the paged variants
// with the verify launches (wmtp_verify.hip) and the ring variants with the
// window launches (wmtp_window.hip).  Instantiating both in one unit changed
// the compiler's instruction schedule of the paged variants.
#pragma once

#include "wmtp_device.hpp"

namespace wmtp {

namespace {

constexpr int kVD = 256;                 // head_dim served by the MFMA verify
constexpr int kVTile = 32;               // keys per tile
constexpr int kVQ = kVD / 4;             // d per wave (64)
constexpr int kVNQ = kVQ * 2 / 16;       // 16-byte pieces per quarter row (8)
constexpr int kVKS = kVQ / 16;           // k-steps per quarter (4)
constexpr int kVStage = kVTile * kVQ * 2;   // bytes of one wave's K stage (4 KiB)
constexpr int kVLoads = kVStage / 1024;  // 16-byte loads per lane per K tile (4)

// Swizzled piece (16 bytes) of logical piece p of key row i (8 pieces per row):
// 8 consecutive keys read by 8 consecutive lanes hit 8 different bank groups.
__device__ __forceinline__ int vpiece(int i, int p) { return i * kVNQ + ((p ^ i) & 7); }

__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

}  // namespace

// A wave's quarter of Q^T for one row tile: lane (packed row c32, half kh),
// k-step s -> piece 2s + kh of the row's quarter; zero for padding rows.  The
// loads are settled here, so none is still pending at the header of the main
// loop (which would force a full drain per tile).
template <int D, int G>
__device__ __forceinline__ void load_q_quarter(u32x4 (&qreg)[kVKS], const SplitArgs& a, int b, int h, int tq,
                                               int rows, int wave, int c32, int kh) {
  constexpr int ROWB = D * 2;
  const uint8_t* q8 = static_cast<const uint8_t*>(a.q);
  const int j = c32;
  const int i = j / G, g = j % G;
  const int64_t qrow = ((int64_t)b * tq + i) * a.num_q_heads + (int64_t)h * G + g;
#pragma unroll
  for (int s = 0; s < kVKS; ++s) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (j < rows) x = *reinterpret_cast<const u32x4*>(q8 + qrow * ROWB + wave * (kVQ * 2) + (2 * s + kh) * 16);
    qreg[s] = x;
  }
#pragma unroll
  for (int s = 0; s < kVKS; ++s) asm volatile("" ::"v"(qreg[s]));
}

// One row tile: t_q x G <= 32 packed rows, two workgroups per CU.  SINGLE: one
// query token (t_q = 1, the draft step); otherwise t_q comes from the
// arguments.  RING (with SINGLE): the windowed draft step, whose keys are the
// visible entries of the compact ring (sinks, then the window) instead of a
// paged context; each lane addresses its keys by ring slot, and a key whose
// slot tag does not hold its position (a hole) is masked.
template <int D, int G, bool SINGLE, bool RING>
__global__ __launch_bounds__(D / kVQ * 64, 8 / (D / kVQ)) void mfma_attn_kernel(const SplitArgs a) {
  static_assert(!RING || SINGLE, "the ring serves the one-query draft step");
  static_assert(D == 64 || D == 128 || D == 256, "head_dim: one, two or four 64-element wave slices");
  constexpr int ROWB = D * 2;
  constexpr int NW = D / kVQ;                // waves, one 64-element slice of D each
  constexpr float TAU = 8.0f;

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[NW * kVStage];
  __shared__ __attribute__((aligned(16))) float sc_lds[2 * NW * 16 * 64];   // [buf][wave][4][lane][4]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads, tq = SINGLE ? 1 : a.t_q;
  const int rows = tq * G;
  const int h = blockIdx.x % Hkv;
  const int sg = blockIdx.x / Hkv;
  const int b = seq_of_split(a, sg);
  const int n = a.seq_len[b];
  // Keys: positions 0..n-1 of the paged context, or the ring's visible entries.
  WindowView wv;
  if constexpr (RING) wv = WindowView(a, b, n);
  const int nkeys = RING ? wv.nvis : n;
  const int t_begin = (sg - a.split_base[b]) * a.chunk;
  const int t_end = min(t_begin + a.chunk, nkeys);
  const int ntiles = (t_end - t_begin + kVTile - 1) / kVTile;
  const int last_blk_idx = (t_end - 1) >> 4;
  if (a.t_new > 0) {
    if constexpr (RING) {
      // one new token at n - 1: the last visible entry, in the sequence's last split
      if (t_end == nkeys) append_own_rows<true>(a, b, h, n, n - 1, n, ROWB);
    } else {
      append_own_rows<false>(a, b, h, n, max(t_begin, n - a.t_new), t_end, ROWB);
    }
  }
  const const_i32_ptr bt_row = as_const_i32(a.block_table) + (int64_t)b * a.bt_stride;
  const int64_t run_bytes = (int64_t)a.run_rows * ROWB;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + wave * (kVQ * 2);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + wave * (kVQ * 2);
  const int64_t ring_seq = RING ? ((int64_t)b * Hkv + h) * a.slots * (int64_t)ROWB : 0;
  const int32_t* tags = a.slot_pos + (RING ? (int64_t)b * a.slots : 0);

  const int c32 = lane & 31;     // key (A rows) / packed query row within a row tile (B, C columns)
  const int kh = lane >> 5;      // which 8-element half of a k-step

  // ---- this wave's quarter of Q^T.  Paged: the query arrives before the first
  // tiles are issued.  Ring: work items are a tile or two long, so the first
  // tiles go out first and the query's latency hides behind theirs.  The paged
  // form writes out the loads of load_q_quarter: calling the helper here
  // changed the compiler's schedule of the paged variants' main loop, and the
  // verify launch measured about 0.6% slower.
  u32x4 qreg[kVKS];
  if constexpr (!RING) {
    const uint8_t* q8 = static_cast<const uint8_t*>(a.q);
    const int j = c32;
    const int i = j / G, g = j % G;
    const int64_t qrow = ((int64_t)b * tq + i) * Hq + (int64_t)h * G + g;
#pragma unroll
    for (int s = 0; s < kVKS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j < rows) x = *reinterpret_cast<const u32x4*>(q8 + qrow * ROWB + wave * (kVQ * 2) + (2 * s + kh) * 16);
      qreg[s] = x;
    }
    // Settle the query loads here, so no load issued before the main loop is
    // still pending at its header (which would force a full drain per tile).
#pragma unroll
    for (int s = 0; s < kVKS; ++s) asm volatile("" ::"v"(qreg[s]));
  }

  uint8_t* my_k = k_lds + wave * kVStage;
  const float c = a.scale_log2;
  // Last key packed row c32 may see in this split (query token c32 / G is causal
  // at n - t_q + c32 / G), and the last key every row sees: only tiles reaching
  // past the latter need a mask.  Padding rows (>= rows) have zero queries and
  // are never written, so they are left unmasked.
  const int row_last = min(n - tq + c32 / G, t_end - 1);
  const int all_last = min(n - tq, t_end - 1);

  // Byte offsets of the two (block, head) runs of 16 keys covering tile `it`.
  // The ring's prefetches past the split's end (never consumed) read the
  // sequence's first tile instead: every work item of the sequence and head
  // asks for the same bytes, which the caches then serve.  The block ids come
  // in through scalar loads one tile before the loads that use them.
  auto tile_runs = [&](int it, int64_t (&run)[2]) {
    const int t0 = it < ntiles ? t_begin + it * kVTile : 0;
    if constexpr (RING) {
      run[0] = run[1] = t0;     // the ring only needs the tile's first entry
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int bi = min((t0 >> 4) + j, last_blk_idx);
        run[j] = paged_block_run(paged_block_uniform(bt_row, (int64_t)bi * kBlock, a.max_block), h, Hkv, run_bytes);
      }
    }
  };

  // Register ring: tile i's K and V arrive in slot i % kRing, issued kRing - 1
  // tiles ahead, so two tiles per wave are in flight while one is computed.
  constexpr int kRing = 3;
  u32x4 kreg[kRing][kVLoads];
  uint32_t vreg[kRing][2][8];
  int32_t tagreg[kRing] = {};
  int64_t run_next[2];

  // K quarter tile: load l of a lane covers stage piece P = 64 l + lane, i.e. key
  // 8 l + lane / 8, piece lane % 8: loads 0, 1 read block run 0 and loads 2, 3
  // run 1, at lane offset k_off (+ 4 KiB for odd l).
  // V: element jj (0..7) of k-step ks for this lane's half is key 16 ks + 8 (jj / 4)
  // + 4 kh + jj % 4 (block run ks); the lane holds d = 2 c32, 2 c32 + 1 of the
  // wave's quarter (one dword), at lane offset v_off + (8 (jj / 4) + jj % 4) rows.
  // K and V are read once per launch: non-temporal loads.
  // Tiles past the end load the sequence's first tile (never consumed), so every
  // body issues the same loads and the loop has no load-carrying branch.  The two
  // 32-bit lane offsets are passed opaque, so they are not widened and hoisted
  // but feed the "uniform base + 32-bit offset" load form directly.
  // Ring: the same keys, each at its own slot of the sequence's ring (entries
  // clamped to the split), and lane c32's tag for the tile's key c32.
  const uint32_t k_off0 = (uint32_t)((lane >> 3) * ROWB + (lane & 7) * 16);
  const uint8_t* kbase_hi = kbase + 8 * ROWB;
  const uint32_t v_off0 = (uint32_t)(4 * kh * ROWB + c32 * 4);
  // Forced inline: the ring's issue step is large enough that the compiler
  // would otherwise call it, indexing the register ring at run time (which
  // demotes it to scratch memory).
  auto issue = [&](int slot, const int64_t (&run)[2], uint32_t k_off, uint32_t v_off) __attribute__((always_inline)) {
    if constexpr (RING) {
      const int t0 = (int)run[0];
      auto row_off = [&](int key) __attribute__((always_inline)) {
        return (uint32_t)wv.slot(min(t0 + key, t_end - 1)) * ROWB;
      };
#pragma unroll
      for (int l = 0; l < kVLoads; ++l)
        kreg[slot][l] = load_nt<u32x4>(kbase + ring_seq, row_off(8 * l + (lane >> 3)) + (lane & 7) * 16);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          vreg[slot][ks][jj] =
              load_nt<uint32_t>(vbase + ring_seq, row_off(16 * ks + 8 * (jj >> 2) + 4 * kh + (jj & 3)) + c32 * 4);
      tagreg[slot] = tags[wv.slot(min(t0 + c32, t_end - 1))];
      (void)k_off;
      (void)v_off;
    } else {
#pragma unroll
      for (int l = 0; l < kVLoads; ++l)
        kreg[slot][l] = load_nt<u32x4>(((l & 1) ? kbase_hi : kbase) + run[l >> 1], k_off);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          vreg[slot][ks][jj] = load_nt<uint32_t>(vbase + run[ks] + (8 * (jj >> 2)) * ROWB, v_off + (jj & 3) * ROWB);
    }
  };

  f32x16 O[2];
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int x = 0; x < 16; ++x) O[e][x] = 0.f;
  // Running maximum M of this lane's row in scaled log2 units (scores times c);
  // both halves of the wave hold the same M for a row.
  float M = kNegInf, l_lane = 0.f;

  auto body = [&](int it, int slot) {
    uint32_t k_off = k_off0, v_off = v_off0;
    asm volatile("" : "+v"(k_off), "+v"(v_off));
    const int t0 = t_begin + it * kVTile;
    issue((slot + kRing - 1) % kRing, run_next, k_off, v_off);
    // Keep the loads in issue order at the top of the body: the load order at
    // the loop latch then matches the prologue's and the wait counts stay exact.
    __builtin_amdgcn_sched_barrier(0);

    // ---- K of this tile -> swizzled LDS stage, then partial S^T over this wave's quarter of D
#pragma unroll
    for (int l = 0; l < kVLoads; ++l) {
      const int P = 64 * l + lane;
      *reinterpret_cast<u32x4*>(my_k + vpiece(P / kVNQ, P % kVNQ) * 16) = kreg[slot][l];
    }
    f32x16 sacc;
#pragma unroll
    for (int x = 0; x < 16; ++x) sacc[x] = 0.f;
#pragma unroll
    for (int s = 0; s < kVKS; ++s) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(my_k + vpiece(c32, 2 * s + kh) * 16);
      sacc = mfma32(ka, qreg[s], sacc);
    }
    float* sc = sc_lds + (it & 1) * (NW * 16 * 64);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 w4 = {sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
      *reinterpret_cast<f32x4*>(sc + ((wave * 4 + q) * 64 + lane) * 4) = w4;
    }
    __syncthreads();
    float s2[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 x = *reinterpret_cast<const f32x4*>(sc + (q * 64 + lane) * 4);
#pragma unroll
      for (int w = 1; w < NW; ++w) x += *reinterpret_cast<const f32x4*>(sc + ((w * 4 + q) * 64 + lane) * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) s2[4 * q + e] = x[e];
    }
    // Block ids of the tile the next body issues: scalar loads placed after the
    // last LDS wait of this body, so they complete behind the softmax and PV.
    __builtin_amdgcn_sched_barrier(0);
    tile_runs(it + kRing, run_next);
    __builtin_amdgcn_sched_barrier(0);

    // ---- mask, lazy row maximum.  Paged: only tiles that reach a causal or
    // split boundary.  Ring: keys past the split and holes, from one ballot of
    // the tile's tags (bit k: key k is visible).
    // Keys no row may see get p = 0, but their values may be any bits (rows past a sequence's
    // end in its last block, ring slots never written or stale), and 0 x NaN is NaN: their V
    // elements are zeroed too.  V element (ks, jj) of this lane is the key of score x = 8 ks + jj.
    if constexpr (RING) {
      const uint32_t live = (uint32_t)__ballot(t0 + c32 < t_end && tagreg[slot] == wv.pos(t0 + c32));
      if (live != 0xffffffffu) {
#pragma unroll
        for (int x = 0; x < 16; ++x) {
          const int key = 8 * (x >> 2) + 4 * kh + (x & 3);
          const bool vis = (live >> key) & 1u;
          s2[x] = vis ? s2[x] : kNegInf;
          vreg[slot][x >> 3][x & 7] = vis ? vreg[slot][x >> 3][x & 7] : 0u;
        }
      }
    } else if (t0 + kVTile - 1 > all_last) {
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const int key = t0 + 8 * (x >> 2) + 4 * kh + (x & 3);
        s2[x] = key <= row_last ? s2[x] : kNegInf;
        vreg[slot][x >> 3][x & 7] = key < t_end ? vreg[slot][x >> 3][x & 7] : 0u;
      }
    }
    float mx = s2[0];
#pragma unroll
    for (int x = 1; x < 16; ++x) mx = fmaxf(mx, s2[x]);
    mx = halves_max(mx) * c;       // c > 0 keeps the order and -inf
    if (__ballot(mx > M + TAU) != 0) {
      const float mn = fmaxf(M, mx);
      const float alpha = (M == kNegInf) ? 0.f : fast_exp2(M - mn);
      M = mn;
      l_lane *= alpha;
      // register x of O holds row 8(x/4) + 4kh + x%4, whose factor sits in that lane
#pragma unroll
      for (int x = 0; x < 16; ++x) {
        const float ar = __shfl(alpha, 8 * (x >> 2) + 4 * kh + (x & 3));
        O[0][x] *= ar;
        O[1][x] *= ar;
      }
    }
    // p = 2^(s c - M); a row with no visible key yet keeps M = -inf and gets p = 0.
    uint32_t pk[8];
    const float negM = M == kNegInf ? 0.f : -M;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float p0 = fast_exp2(fmaf(s2[2 * q], c, negM));
      const float p1 = fast_exp2(fmaf(s2[2 * q + 1], c, negM));
      pk[q] = pack_bf16x2(p0, p1);
      l_lane = dot2_bf16(pk[q], kBf16One2, l_lane);   // normaliser from the same bf16 weights
    }

    // ---- O += P V over this wave's quarter of D (2 output tiles, 2 k-steps of 16 keys)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const u32x4 pa = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        u32x4 vb;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          vb[q] = __builtin_amdgcn_perm(vreg[slot][ks][2 * q + 1], vreg[slot][ks][2 * q],
                                        e ? 0x07060302u : 0x05040100u);
        O[e] = mfma32(pa, vb, O[e]);
      }
    }
  };

  // kRing bodies per trip over fixed slots, the last tiles after the loop.  With
  // a single exit the loads pending at the loop header are the same from the
  // prologue and from the latch, so every body waits for its own tile only
  // (early exits inside the trip made the compiler drain one tile more).
  if (ntiles > 0) {
#pragma unroll
    for (int i = 0; i < kRing - 1; ++i) {
      tile_runs(i, run_next);
      issue(i, run_next, k_off0, v_off0);
      // tile by tile, in the order the loop issues them (exact wait counts)
      __builtin_amdgcn_sched_barrier(0);
    }
    tile_runs(kRing - 1, run_next);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (RING) load_q_quarter<D, G>(qreg, a, b, h, tq, rows, wave, c32, kh);
    int it = 0;
    for (; it + 3 <= ntiles; it += 3) {
      body(it, 0);
      body(it + 1, 1);
      body(it + 2, 2);
    }
    if (it < ntiles) body(it, 0);
    if (it + 1 < ntiles) body(it + 1, 1);
  }

  // ---- normalise and write this wave's quarter of every live row
  const float l_row = halves_sum(l_lane);       // lanes c32 and c32 + 32 share a row
  const float inv_row = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int row = 8 * (x >> 2) + 4 * kh + (x & 3);
    const float inv = __shfl(inv_row, row);
    if (row < rows) {
      const int i = row / G, g = row % G;
      const int64_t orow = (int64_t)sg * (tq * Hq) + (int64_t)i * Hq + (int64_t)h * G + g;
      float2 w2;
      w2.x = O[0][x] * inv;
      w2.y = O[1][x] * inv;
      *reinterpret_cast<float2*>(a.part_o + orow * D + wave * kVQ + 2 * c32) = w2;
    }
  }
  if (wave == 0 && lane < rows && lane < 32) {
    const int row = lane;
    const int i = row / G, g = row % G;
    const int64_t orow = (int64_t)sg * (tq * Hq) + (int64_t)i * Hq + (int64_t)h * G + g;
    a.part_lse[orow] = l_row > 0.f ? (M + __log2f(l_row)) * kLn2 : kNegInf;
  }
}

}  // namespace wmtp

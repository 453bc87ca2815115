// Two or three row tiles of verify (33..96 packed rows per KV head) on two wave
// teams: the kernel template, with its row-tile helpers.  Instantiated for
// head_dim 256 with the verify launches (wmtp_verify.hip) and for head_dim 64
// and 128 apart from them (wmtp_verify_small.hip).  The pages' verify is full
// attention of the gamma + 1 drafted positions ("Windowed-MTP: Removing the
// Full-Context Draft-KV Tax at Million-Token Context", arxivlens summary,
// Abstract); packing gamma + 1 > 4 tokens of 8 query heads takes more rows than
// one matrix-core tile holds.
#pragma once

#include "wmtp_row_tile.hpp"

namespace wmtp {

// One row tile of one wave in the two-team kernel: the queries of the
// NQ quarters of D the wave covers (quarters q0 .. q0 + NQ - 1), the row
// tile's softmax state and the wave's accumulators (32 rows x 32 d per
// quarter half).
template <int NQ>
struct RowTile {
  u32x4 q[NQ][kVKS];
  f32x16 O[NQ][2];
  float M, l;
  int row0, row_last, q0;
};

// What a wave of a two-team work item needs to know about it.
struct WorkItem {
  const SplitArgs* a;
  int lane, c32, kh;
  int b, h, sg, n, tq, rows, t_end, all_last;
  float c;                      // score scale in log2 units
};

constexpr int kPart = 4 * 64 * 4;   // floats of one wave's partial S^T tile (16 per lane)

// Queries of row tile r (packed rows 32 r ..), quarters q0 .. q0 + NQ - 1, and a cleared state.
template <int D, int G, int NQ>
__device__ __forceinline__ void init_row_tile(const WorkItem& w, RowTile<NQ>& rt, int r, int q0) {
  constexpr int ROWB = D * 2;
  rt.row0 = 32 * r;
  rt.q0 = q0;
  const uint8_t* q8 = static_cast<const uint8_t*>(w.a->q);
  const int j = rt.row0 + w.c32;
  const int i = j / G, g = j % G;
  const int64_t qrow = ((int64_t)w.b * w.tq + i) * w.a->num_q_heads + (int64_t)w.h * G + g;
#pragma unroll
  for (int hq = 0; hq < NQ; ++hq)
#pragma unroll
    for (int s = 0; s < kVKS; ++s) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (j < w.rows)
        x = *reinterpret_cast<const u32x4*>(q8 + qrow * ROWB + (q0 + hq) * (kVQ * 2) + (2 * s + w.kh) * 16);
      rt.q[hq][s] = x;
    }
#pragma unroll
  for (int hq = 0; hq < NQ; ++hq)
#pragma unroll
    for (int s = 0; s < kVKS; ++s) asm volatile("" ::"v"(rt.q[hq][s]));
  rt.row_last = min(w.n - w.tq + j / G, w.t_end - 1);
#pragma unroll
  for (int hq = 0; hq < NQ; ++hq)
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int x = 0; x < 16; ++x) rt.O[hq][e][x] = 0.f;
  rt.M = kNegInf;
  rt.l = 0.f;
}

// Partial S^T of one row tile over the wave's quarters of D, K from one tile's stage.
template <int NQ>
__device__ __forceinline__ f32x16 qk_partial(const WorkItem& w, const uint8_t* kstage, const RowTile<NQ>& rt) {
  f32x16 sacc;
#pragma unroll
  for (int x = 0; x < 16; ++x) sacc[x] = 0.f;
#pragma unroll
  for (int hq = 0; hq < NQ; ++hq) {
    const uint8_t* kst = kstage + (rt.q0 + hq) * kVStage;
#pragma unroll
    for (int s = 0; s < kVKS; ++s) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(kst + vpiece(w.c32, 2 * s + w.kh) * 16);
      sacc = mfma32(ka, rt.q[hq][s], sacc);
    }
  }
  return sacc;
}

__device__ __forceinline__ void store_partial(const WorkItem& w, const f32x16& sacc, float* part) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 w4 = {sacc[4 * q], sacc[4 * q + 1], sacc[4 * q + 2], sacc[4 * q + 3]};
    *reinterpret_cast<f32x4*>(part + (q * 64 + w.lane) * 4) = w4;
  }
}

__device__ __forceinline__ f32x4 load_partial(const WorkItem& w, const float* part, int q) {
  return *reinterpret_cast<const f32x4*>(part + (q * 64 + w.lane) * 4);
}

// S of a row tile whose D halves are split over a pair of waves: own partial plus the
// partner's.  Addition is commutative, so both waves of the pair get identical scores.
__device__ __forceinline__ void sum2_partials(const WorkItem& w, const f32x16& own, const float* other,
                                              float (&s2)[16]) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const f32x4 x = load_partial(w, other, q);
#pragma unroll
    for (int e = 0; e < 4; ++e) s2[4 * q + e] = own[4 * q + e] + x[e];
  }
}

// Mask, lazy maximum, bf16 weights and O += P V for the tile starting at key t0.
// V comes from the tile's LDS stage (layout [quarter][piece][lane]: piece 2 ks
// and 2 ks + 1 hold the lane's 8 dwords of k-step ks) for the wave's NQ
// quarters q0 ..; key pairs are regrouped here.  Up to two quarters the V
// operands are read before the softmax, so the LDS reads overlap it; a wave
// that covers all of D reads them one quarter at a time during PV (four
// quarters' operands do not fit in its registers beside the accumulators).
template <int NQ>
__device__ __forceinline__ void softmax_pv(const WorkItem& w, int t0, float (&s2)[16], const u32x4 (*vst)[4][64],
                                           RowTile<NQ>& rt) {
  constexpr float TAU = 8.0f;
  constexpr bool kEarlyV = NQ <= 2;
  u32x4 vpre[kEarlyV ? NQ : 1][4];
  if constexpr (kEarlyV) {
#pragma unroll
    for (int hq = 0; hq < NQ; ++hq)
#pragma unroll
      for (int pc = 0; pc < 4; ++pc) vpre[hq][pc] = vst[rt.q0 + hq][pc][w.lane];
  }
  if (t0 + kVTile - 1 > w.all_last) {
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const int key = t0 + 8 * (x >> 2) + 4 * w.kh + (x & 3);
      s2[x] = key <= rt.row_last ? s2[x] : kNegInf;
    }
  }
  float mx = s2[0];
#pragma unroll
  for (int x = 1; x < 16; ++x) mx = fmaxf(mx, s2[x]);
  mx = halves_max(mx) * w.c;
  if (__ballot(mx > rt.M + TAU) != 0) {
    const float mn = fmaxf(rt.M, mx);
    const float alpha = (rt.M == kNegInf) ? 0.f : fast_exp2(rt.M - mn);
    rt.M = mn;
    rt.l *= alpha;
#pragma unroll
    for (int x = 0; x < 16; ++x) {
      const float ar = __shfl(alpha, 8 * (x >> 2) + 4 * w.kh + (x & 3));
#pragma unroll
      for (int hq = 0; hq < NQ; ++hq) {
        rt.O[hq][0][x] *= ar;
        rt.O[hq][1][x] *= ar;
      }
    }
  }
  const float negM = rt.M == kNegInf ? 0.f : -rt.M;
  uint32_t pk[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const float p0 = fast_exp2(fmaf(s2[2 * q], w.c, negM));
    const float p1 = fast_exp2(fmaf(s2[2 * q + 1], w.c, negM));
    pk[q] = pack_bf16x2(p0, p1);
    rt.l = dot2_bf16(pk[q], kBf16One2, rt.l);
  }
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const u32x4 pa = {pk[4 * ks], pk[4 * ks + 1], pk[4 * ks + 2], pk[4 * ks + 3]};
#pragma unroll
    for (int hq = 0; hq < NQ; ++hq) {
      const u32x4 v0 = kEarlyV ? vpre[hq][2 * ks] : vst[rt.q0 + hq][2 * ks][w.lane];
      const u32x4 v1 = kEarlyV ? vpre[hq][2 * ks + 1] : vst[rt.q0 + hq][2 * ks + 1][w.lane];
      const uint32_t vv[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        u32x4 vb;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          vb[q] = __builtin_amdgcn_perm(vv[2 * q + 1], vv[2 * q], e ? 0x07060302u : 0x05040100u);
        rt.O[hq][e] = mfma32(pa, vb, rt.O[hq][e]);
      }
    }
  }
}

// Normalise and write the wave's quarters of the row tile's live rows; the lse
// comes from the wave that covers quarter 0.
template <int D, int G, int NQ>
__device__ __forceinline__ void finish_row_tile(const WorkItem& w, const RowTile<NQ>& rt) {
  const SplitArgs& a = *w.a;
  const int Hq = a.num_q_heads;
  const float l_row = halves_sum(rt.l);
  const float inv_row = l_row > 0.f ? 1.f / l_row : 0.f;
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int rl = 8 * (x >> 2) + 4 * w.kh + (x & 3);
    const float inv = __shfl(inv_row, rl);
    const int row = rt.row0 + rl;
    if (row < w.rows) {
      const int i = row / G, g = row % G;
      const int64_t orow = (int64_t)w.sg * (w.tq * Hq) + (int64_t)i * Hq + (int64_t)w.h * G + g;
#pragma unroll
      for (int hq = 0; hq < NQ; ++hq) {
        float2 w2;
        w2.x = rt.O[hq][0][x] * inv;
        w2.y = rt.O[hq][1][x] * inv;
        *reinterpret_cast<float2*>(a.part_o + orow * D + (rt.q0 + hq) * kVQ + 2 * w.c32) = w2;
      }
    }
  }
  if (rt.q0 == 0 && w.lane < 32 && rt.row0 + w.lane < w.rows) {
    const int row = rt.row0 + w.lane;
    const int i = row / G, g = row % G;
    const int64_t orow = (int64_t)w.sg * (w.tq * Hq) + (int64_t)i * Hq + (int64_t)w.h * G + g;
    a.part_lse[orow] = l_row > 0.f ? (rt.M + __log2f(l_row)) * kLn2 : kNegInf;
  }
}

// The paged K/V loads of one wave's quarter of D, issued kRing - 1 tiles ahead
// into a register ring exactly as in the one-row-tile kernel (the two-team
// kernel's loader team).
struct QuarterLoader {
  static constexpr int kRing = 3;
  u32x4 kreg[kRing][kVLoads];
  uint32_t vreg[kRing][2][8];
};

// Two or three row tiles (33..96 packed rows) on two teams of 4 waves, 512
// threads.  With all row tiles in one wave the per-tile chain of LDS stages,
// barriers, MFMA and softmax has nothing to hide behind at one wave per SIMD;
// here team 0 loads K and V exactly as the one-row-tile kernel and stages both
// in LDS, while team 1 computes tile t - 1 from those stages: every SIMD runs
// one wave of each team, and HBM is read once.
//   RT = 2: team 1's waves form two pairs, one per row tile; each wave covers
//   half of D, so it contracts its row tile over two quarters of D, runs one
//   row tile's softmax and adds its partner's partial score tile to its own.
//   Both waves of a pair add the same two partials (addition is commutative),
//   so they hold identical weights.
//   RT = 3: waves 0..2 of team 1 each take one row tile over all of D (16
//   MFMAs for S, 16 for PV per tile), so no partial scores are exchanged and
//   each row tile's softmax runs once; wave 3 only keeps the barrier count.
// One barrier per tile step: the K/V stages rotate over three buffers and the
// pairs' score exchange over two; neither team can pass a step's barrier
// before the other reaches it, so team 0 rewrites a stage only after team 1
// has passed the barrier that follows its last read of it.
template <int D, int G, int RT>
__global__ __launch_bounds__((D / kVQ + 4) * 64, 1) void mfma_attn_teams_kernel(const SplitArgs a) {
  static_assert(RT == 2 || RT == 3, "two or three row tiles");
  static_assert(D == 64 || D == 128 || D == 256, "head_dim: one, two or four 64-element slices");
  constexpr int ROWB = D * 2;
  constexpr int NW = D / kVQ;                  // loader waves (team 0), one slice of D each
  // Team 1 takes one row tile per wave over all of D, except two row tiles at
  // head_dim 256, which go to pairs of waves over half of D each.
  constexpr bool kPairs = RT == 2 && D == 256;
  constexpr int NB = 3;                        // K/V stage buffers
  constexpr int NP = 2;                        // score-exchange buffers (pairs)

  __shared__ __attribute__((aligned(16))) uint8_t k_stage[NB][NW * kVStage];   // [tile % NB][slice]
  __shared__ __attribute__((aligned(16))) u32x4 v_stage[NB][NW][4][64];        // [tile % NB][slice][piece][lane]
  __shared__ __attribute__((aligned(16))) float sc_lds[NP][kPairs ? 4 * kPart : 1];   // [tile % NP][wave partial]

  WorkItem w;
  w.a = &a;
  w.lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int team, wave;                              // team 0: waves 0 .. NW-1; team 1: the next 4
  if constexpr (NW == 4) {
    team = wid >> 2;
    wave = wid & 3;
  } else {
    team = wid < NW ? 0 : 1;
    wave = wid < NW ? wid : wid - NW;
  }
  const int Hkv = a.num_kv_heads;
  w.tq = a.t_q;
  w.rows = w.tq * G;
  w.h = blockIdx.x % Hkv;
  w.sg = blockIdx.x / Hkv;
  w.b = seq_of_split(a, w.sg);
  w.n = a.seq_len[w.b];
  const int t_begin = (w.sg - a.split_base[w.b]) * a.chunk;
  w.t_end = min(t_begin + a.chunk, w.n);
  const int ntiles = (w.t_end - t_begin + kVTile - 1) / kVTile;
  const int last_blk_idx = (w.t_end - 1) >> 4;
  if (a.t_new > 0) append_own_rows<false>(a, w.b, w.h, w.n, max(t_begin, w.n - a.t_new), w.t_end, ROWB);
  const const_i32_ptr bt_row = as_const_i32(a.block_table) + (int64_t)w.b * a.bt_stride;
  const int64_t run_bytes = (int64_t)a.run_rows * ROWB;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + wave * (kVQ * 2);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + wave * (kVQ * 2);
  const int lane = w.lane;
  w.c32 = lane & 31;
  w.kh = lane >> 5;
  w.c = a.scale_log2;
  w.all_last = min(w.n - w.tq, w.t_end - 1);
  const int c32 = w.c32, kh = w.kh;

  if (team == 0) {
    // ---- loader team: the one-row-tile kernel's loads and ring, staged for team 1
    auto tile_runs = [&](int it, int64_t (&run)[2]) {
      const int t0 = it < ntiles ? t_begin + it * kVTile : 0;     // past the end: the sequence's first tile
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int bi = min((t0 >> 4) + j, last_blk_idx);
        run[j] = paged_block_run(paged_block_uniform(bt_row, (int64_t)bi * kBlock, a.max_block), w.h, Hkv,
                                 run_bytes);
      }
    };
    constexpr int kRing = QuarterLoader::kRing;
    QuarterLoader ld;
    int64_t run_next[2];
    const uint32_t k_off0 = (uint32_t)((lane >> 3) * ROWB + (lane & 7) * 16);
    const uint8_t* kbase_hi = kbase + 8 * ROWB;
    const uint32_t v_off0 = (uint32_t)(4 * kh * ROWB + c32 * 4);
    auto issue = [&](int slot, const int64_t (&run)[2], uint32_t k_off, uint32_t v_off) {
#pragma unroll
      for (int l = 0; l < kVLoads; ++l)
        ld.kreg[slot][l] = load_nt<u32x4>(((l & 1) ? kbase_hi : kbase) + run[l >> 1], k_off);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
          ld.vreg[slot][ks][jj] = load_nt<uint32_t>(vbase + run[ks] + (8 * (jj >> 2)) * ROWB, v_off + (jj & 3) * ROWB);
    };
    auto body = [&](int it, int slot) {
      uint32_t k_off = k_off0, v_off = v_off0;
      asm volatile("" : "+v"(k_off), "+v"(v_off));
      issue((slot + kRing - 1) % kRing, run_next, k_off, v_off);
      __builtin_amdgcn_sched_barrier(0);
      uint8_t* kst = k_stage[it % NB] + wave * kVStage;
#pragma unroll
      for (int l = 0; l < kVLoads; ++l) {
        const int P = 64 * l + lane;
        *reinterpret_cast<u32x4*>(kst + vpiece(P / kVNQ, P % kVNQ) * 16) = ld.kreg[slot][l];
      }
      // Keys past the split's end get p = 0, but rows past the sequence's end may hold any bits
      // (0 x NaN is NaN): on the tile that reaches past it, their values are staged as zeros.
      // Element jj of k-step ks is key 16 ks + 8 (jj / 4) + 4 kh + jj % 4 of the tile.
      const int t0 = t_begin + it * kVTile;
      const bool tail = t0 + kVTile > w.t_end;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x4 v4 = {ld.vreg[slot][q >> 1][4 * (q & 1)], ld.vreg[slot][q >> 1][4 * (q & 1) + 1],
                    ld.vreg[slot][q >> 1][4 * (q & 1) + 2], ld.vreg[slot][q >> 1][4 * (q & 1) + 3]};
        if (tail) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int jj = 4 * (q & 1) + e;
            const int key = t0 + 16 * (q >> 1) + 8 * (jj >> 2) + 4 * kh + (jj & 3);
            v4[e] = key < w.t_end ? v4[e] : 0u;
          }
        }
        v_stage[it % NB][wave][q][lane] = v4;
      }
      __syncthreads();
      tile_runs(it + kRing, run_next);
      __builtin_amdgcn_sched_barrier(0);
    };
    if (ntiles > 0) {
#pragma unroll
      for (int i = 0; i < kRing - 1; ++i) {
        tile_runs(i, run_next);
        issue(i, run_next, k_off0, v_off0);
        __builtin_amdgcn_sched_barrier(0);
      }
      tile_runs(kRing - 1, run_next);
      __builtin_amdgcn_sched_barrier(0);
      int it = 0;
      for (; it + 3 <= ntiles; it += 3) {
        body(it, 0);
        body(it + 1, 1);
        body(it + 2, 2);
      }
      if (it < ntiles) body(it, 0);
      if (it + 1 < ntiles) body(it + 1, 1);
    }
    // team 1 still computes the last tile: its barrier
    __syncthreads();
  } else if constexpr (!kPairs) {
    // ---- team 1: wave r < RT takes row tile r of tile it - 1 over all of D
    if (wave < RT) {
      RowTile<NW> rt;
      init_row_tile<D, G>(w, rt, wave, 0);
      for (int it = 0; it <= ntiles; ++it) {
        const int t = it - 1;
        f32x16 sacc;
        if (t >= 0) sacc = qk_partial(w, k_stage[t % NB], rt);
        __syncthreads();
        if (t >= 0) {
          float s2[16];
#pragma unroll
          for (int x = 0; x < 16; ++x) s2[x] = sacc[x];
          softmax_pv(w, t_begin + t * kVTile, s2, v_stage[t % NB], rt);
        }
      }
      finish_row_tile<D, G>(w, rt);
    } else {
      for (int it = 0; it <= ntiles; ++it) __syncthreads();
    }
  } else {
    // ---- team 1, two row tiles: waves 2r and 2r + 1 take row tile r of tile it - 1,
    // each over one half of D (quarters 2 dh and 2 dh + 1)
    const int r = wave >> 1, dh = wave & 1;
    RowTile<2> rt;
    init_row_tile<D, G>(w, rt, r, 2 * dh);
    for (int it = 0; it <= ntiles; ++it) {
      const int t = it - 1;
      float* parts = sc_lds[it % NP] + 2 * r * kPart;      // the pair's two partials
      f32x16 own;
      if (t >= 0) {
        own = qk_partial(w, k_stage[t % NB], rt);
        store_partial(w, own, parts + dh * kPart);
      }
      __syncthreads();
      if (t >= 0) {
        float s2[16];
        sum2_partials(w, own, parts + (dh ^ 1) * kPart, s2);
        softmax_pv(w, t_begin + t * kVTile, s2, v_stage[t % NB], rt);
      }
    }
    finish_row_tile<D, G>(w, rt);
  }
}

}  // namespace wmtp

// Split-K flash-decoding for the MTP draft head on gfx950, with fp32 softmax
// weights in the PV product: the slice kernel.
//
// The native MTP draft attends over the whole KV cache at every draft step, so
// its read scales with the context length; Windowed-MTP attends over sink tokens
// plus a window of recent tokens held in a compact ring ("Windowed-MTP:
// Removing the Full-Context Draft-KV Tax at Million-Token Context", arxivlens
// summary, Abstract; readpriors.com post, What happened).  This kernel serves
// window mode (bf16 or fp32 data) and full mode with fp32 data; the two differ
// only in how a visible entry is located (block table vs ring slot + tag
// check).  Full mode in bf16 runs on the whole-tile kernel (wmtp_draft_rows.hip)
// and bf16 PV weights on the matrix-core kernels.  Window mode walks the visible
// positions (the sequence's own sinks, then its window) and reads each from its
// ring slot, so its cost follows the sequence's S_b + W_b, not the ring's size.
//
// Work item = (sequence b, KV head h, split of `chunk` visible entries); one
// workgroup per item whose waves each own a 64-byte slice of every K/V row (8
// waves for a 512-byte bf16 row of head_dim 256).  The G query heads of the KV
// head are packed, so each K/V byte is read from HBM once per group.
//
// Per 64-entry tile:
//   1. K: every wave loads its slice of the 64 rows (coalesced 16-byte loads
//      into registers, two tiles ahead) and at the start of the tile stores it
//      into a wave-private LDS stage whose 16-byte pieces are XOR-swizzled so
//      that "one lane per entry" reads are free of bank conflicts.
//   2. QK: lane = entry; the wave's slice of the G query rows comes from
//      SGPRs (wave-uniform scalar loads), so bf16 pairs go straight into
//      v_dot2_f32_bf16 with no unpacking and no cross-lane reduction.
//   3. The slice dot products are summed through LDS (one barrier per tile).
//   4. Online softmax in the log2 domain with a lazy maximum: the running max is
//      only raised (and the accumulators rescaled) when a score exceeds it by
//      more than 2^8, which is rare after the first tile; the result is the same
//      up to rounding because numerator and denominator share the reference.
//   5. PV: each wave owns its slice of D; V rows arrive in registers two tiles
//      ahead; probabilities are handed from the entry lanes through LDS.
// In full mode K and V go through a 3-slot register ring; the loop body is
// unrolled over the slots and every body issues the same loads, so the
// compiler's wait counts keep two tiles in flight.  Window mode's work items
// read one or a few tiles and use a single slot.
// The split writes o = sum p v / sum p and lse = ln sum exp(s) for every packed
// row; a separate LSE combine merges the splits.
#include "wmtp_device.hpp"
#include "wmtp_launch.hpp"

namespace wmtp {

template <int D, int G, bool BF16>
struct DraftShape {
  static constexpr int ES = BF16 ? 2 : 4;      // element bytes
  static constexpr int ROWB = D * ES;          // bytes of one entry's row (one head)
  // Each wave owns a slice of QB bytes of every row: 64 bytes (4 waves for a
  // 256-byte row, 8 for 512, 16 for 1 KiB), or a quarter of shorter rows.
  static constexpr int QB = ROWB >= 256 ? 64 : ROWB / 4;
  static constexpr int NW = ROWB / QB;         // waves per workgroup
  static constexpr int THREADS = NW * 64;
  static constexpr int NCH = QB / 16;          // 16-byte pieces per row slice
  static constexpr int EPP = 16 / ES;          // elements per piece
  static constexpr int TILE = 64;
  static constexpr int TPI = 64 / NCH;         // entries covered by one 1 KiB wave load
  static constexpr int GP = (G + 3) / 4 * 4;   // G padded to whole float4 planes
  static constexpr int KSTAGE = TILE * QB;     // bytes of one wave's K stage
  static constexpr int LDS_BYTES = NW * KSTAGE + 2 * NW * GP * TILE * 4;
  // PV layout: each lane loads 8 bytes of a V row per load (EV elements);
  // LPR lanes cover one row slice, TPV entries per wave load, NV loads per tile.
  static constexpr int VB = 8;
  static constexpr int EV = VB / ES;
  static constexpr int LPR = QB / VB;
  static constexpr int TPV = 64 / LPR;
  static constexpr int NV = TILE / TPV;
  static_assert(NCH >= 2 && NCH <= 16, "a row slice must hold 2..16 pieces");
  static_assert(GP * TILE * 4 <= KSTAGE, "probability tile must fit in a K stage");
};

// Physical 16-byte piece of logical piece c of tile entry t in a wave's K stage.
// Entry t owns NCH consecutive pieces; 8 consecutive entries read by 8
// consecutive lanes land in 8 different bank groups (one 128-byte bank sweep).
template <int NCH>
__device__ __forceinline__ int k_piece(int t, int c) {
  if constexpr (NCH >= 8) {
    return t * NCH + ((c & ~7) | ((c ^ t) & 7));
  } else {
    constexpr int per_sweep = 8 / NCH;            // entries sharing one 128-byte sweep
    return t * NCH + (c ^ ((t / per_sweep) % NCH));
  }
}

template <int D, int G, bool BF16, bool WINDOW>
__global__ __launch_bounds__((DraftShape<D, G, BF16>::THREADS)) void draft_splitk_kernel(const SplitArgs a) {
  using S = DraftShape<D, G, BF16>;
  constexpr int NCH = S::NCH, TPI = S::TPI, GP = S::GP, QB = S::QB, ROWB = S::ROWB, NW = S::NW;
  constexpr int EV = S::EV, LPR = S::LPR, TPV = S::TPV, NV = S::NV;
  constexpr float TAU = 8.0f;   // lazy-max slack, log2 units

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[NW * S::KSTAGE];
  __shared__ __attribute__((aligned(16))) float sc_lds[2 * NW * GP * S::TILE];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = a.num_kv_heads;
  const int h = blockIdx.x % Hkv;
  const int sg = blockIdx.x / Hkv;
  const int b = seq_of_split(a, sg);
  const int n = a.seq_len[b];
  // Window mode reads the visible set in position order (sinks, then the window).
  const WindowView wv(a, b, n);
  const int nvis = WINDOW ? wv.nvis : n;
  const int t_begin = (sg - a.split_base[b]) * a.chunk;
  const int t_end = min(t_begin + a.chunk, nvis);
  const int ntiles = (t_end - t_begin + S::TILE - 1) / S::TILE;
  if (a.t_new > 0) {
    if constexpr (WINDOW) {
      // one new token at n - 1: the last visible entry, in the sequence's last split
      if (t_end == nvis) append_own_rows<true>(a, b, h, n, n - 1, n, ROWB);
    } else {
      append_own_rows<false>(a, b, h, n, max(t_begin, n - a.t_new), t_end, ROWB);
    }
  }

  const uint8_t* kbase = static_cast<const uint8_t*>(a.k) + wave * QB;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v) + wave * QB;
  const const_i32_ptr bt_row = as_const_i32(a.block_table) + (int64_t)b * a.bt_stride;
  const int64_t ring_seq = ((int64_t)b * Hkv + h) * a.slots * (int64_t)ROWB;
  const int32_t* tags = a.slot_pos + (int64_t)b * a.slots;
  const int last_blk_idx = (t_end - 1) >> 4;

  // query rows of this KV head, this wave's slice of D (wave-uniform -> SGPRs)
  const int64_t qrow0 = (int64_t)b * a.num_q_heads + (int64_t)h * G;
  const_u32_ptr q32 = as_const_u32(a.q) + qrow0 * (D * S::ES / 4) + wave * (QB / 4);

  uint8_t* my_k = k_lds + wave * S::KSTAGE;

  // ---- addressing.  A tile's entries live in up to 4 runs of 16 rows (paged);
  // in the ring every lane adds its entry's slot offset to the ring's base.
  // run[j] is the uniform byte offset of run j; a lane adds a 32-bit offset.
  // Entries past the split end are clamped to a valid row.
  auto tile_runs = [&](int t0, int64_t (&run)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (WINDOW) {
        run[j] = ring_seq;
      } else {
        const int bi = min((t0 >> 4) + j, last_blk_idx);
        run[j] = paged_block_run(paged_block_uniform(bt_row, (int64_t)bi * kBlock, a.max_block), h, Hkv,
                                 (int64_t)a.run_rows * ROWB);
      }
    }
  };
  auto lane_off = [&](int t0, int tt) -> uint32_t {
    if constexpr (WINDOW) return (uint32_t)wv.slot(min(t0 + tt, t_end - 1)) * ROWB;
    return (uint32_t)(tt & 15) * ROWB;
  };
  auto run_base = [&](const uint8_t* base, const int64_t (&run)[4], int first, int span, int tt) -> const uint8_t* {
    if constexpr (WINDOW) return base + run[0];
    if (span <= 16) return base + run[first >> 4];
    const int j = tt >> 4;                      // entries of one load straddle blocks
    int64_t r = run[0];
    r = j == 1 ? run[1] : r;
    r = j == 2 ? run[2] : r;
    r = j == 3 ? run[3] : r;
    return base + r;
  };

  // Ordinary loads, also for the paged pool: each wave reads a 64-byte half of
  // 128-byte lines whose other half another wave reads, and non-temporal loads
  // (which the matrix-core kernel uses) measured 10% slower here.
  // Register ring: the K and V of tile i arrive in slot i % kRing, issued
  // kRing - 1 tiles ahead, so two tiles per wave are in flight while one is
  // computed.  Window mode reads one or a few tiles per work item (its splits
  // are short so that many work items cover the ring at once): a single slot,
  // a third of the code on that latency-bound path.
  constexpr int kRing = WINDOW ? 1 : 3;
  u32x4 kreg[kRing][NCH];
  uint2 vreg[kRing][NV];
  int tag[kRing] = {};

  // Loads of tile `it`; every body issues the same number of loads.  The ring's
  // prefetches past the split's end (full mode, never consumed) read the
  // sequence's first tile, the same bytes for every work item of the sequence
  // and head, which the caches then serve.  `ln` is this lane's index.
  auto issue = [&](int it, int slot, int ln) {
    const int t0 = it < ntiles ? t_begin + it * S::TILE : 0;
    int64_t run[4];
    tile_runs(t0, run);
    const int k_tok = ln / NCH, k_c = ln % NCH;
    const int v_tok = ln / LPR, v_d = ln % LPR;
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int tt = i * TPI + k_tok;
      kreg[slot][i] = load_at<u32x4>(run_base(kbase, run, i * TPI, TPI, tt), lane_off(t0, tt) + k_c * 16);
    }
    // V: load k brings entry k*TPV + v_tok, bytes [8 v_d, 8 v_d + 8) of the slice.
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int tt = k * TPV + v_tok;
      vreg[slot][k] = load_at<uint2>(run_base(vbase, run, k * TPV, TPV, tt), lane_off(t0, tt) + v_d * 8);
    }
    if constexpr (WINDOW) tag[slot] = tags[wv.slot(min(t0 + ln, t_end - 1))];
  };

  float o[G][EV];
  float l_lane[G], M[G];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    l_lane[g] = 0.f;
    M[g] = kNegInf;
#pragma unroll
    for (int e = 0; e < EV; ++e) o[g][e] = 0.f;
  }

  auto body = [&](int it, int slot) {
    int ln = lane;
    asm volatile("" : "+v"(ln));     // recompute lane offsets per tile instead of holding them
    const int t0 = t_begin + it * S::TILE;
    issue(it + kRing - 1, (slot + kRing - 1) % kRing, ln);
    __builtin_amdgcn_sched_barrier(0);   // loads stay in issue order at the top of the body
    const int k_tok = ln / NCH, k_c = ln % NCH;
    const int v_tok = ln / LPR;

    // ---- K of this tile -> swizzled LDS stage
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      *reinterpret_cast<u32x4*>(my_k + k_piece<NCH>(i * TPI + k_tok, k_c) * 16) = kreg[slot][i];

    // ---- QK: lane = entry, partial dot over this wave's slice of D
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
    // q is re-read from the scalar cache every tile: hoisting it out of the loop
    // would hold all of the wave's slice of the G query rows in registers.
    const_u32_ptr qt = q32;
    asm volatile("" : "+s"(qt));
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4 kk = *reinterpret_cast<const u32x4*>(my_k + k_piece<NCH>(ln, c) * 16);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const_u32_ptr qg = qt + (int64_t)g * (D * S::ES / 4) + c * 4;
        if constexpr (BF16) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[g] = dot2_bf16(qg[e], kk[e], acc[g]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[g] = fmaf(__uint_as_float(qg[e]), __uint_as_float(kk[e]), acc[g]);
        }
      }
    }

    // ---- sum the NW slice products through LDS
    float* sc = sc_lds + (it & 1) * (NW * GP * S::TILE);
#pragma unroll
    for (int pl = 0; pl < GP / 4; ++pl) {
      f32x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (pl * 4 + e < G) ? acc[pl * 4 + e] : 0.f;
      *reinterpret_cast<f32x4*>(sc + ((wave * (GP / 4) + pl) * S::TILE + ln) * 4) = w4;
    }
    __syncthreads();
    float s2[G];
#pragma unroll
    for (int g = 0; g < G; ++g) s2[g] = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
#pragma unroll
      for (int pl = 0; pl < GP / 4; ++pl) {
        const f32x4 w4 = *reinterpret_cast<const f32x4*>(sc + ((w * (GP / 4) + pl) * S::TILE + ln) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (pl * 4 + e < G) s2[pl * 4 + e] += w4[e];
      }
    }

    // ---- online softmax (log2 domain, lazy maximum)
    bool valid = t0 + ln < t_end;
    // the slot must hold exactly the entry's position (a hole or a stale entry is masked)
    if constexpr (WINDOW) valid = valid && tag[slot] == wv.pos(t0 + ln);
    bool exceed = false;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      s2[g] = valid ? s2[g] * a.scale_log2 : kNegInf;
      exceed = exceed || (s2[g] > M[g] + TAU);
    }
    if (__ballot(exceed) != 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mt = wave_max(s2[g]);
        const float mn = fmaxf(M[g], mt);
        const float alpha = (M[g] == kNegInf) ? 0.f : exp2f(M[g] - mn);
        M[g] = mn;
        l_lane[g] *= alpha;
#pragma unroll
        for (int e = 0; e < EV; ++e) o[g][e] *= alpha;
      }
    }
    float p[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      p[g] = valid ? exp2f(s2[g] - M[g]) : 0.f;
      l_lane[g] += p[g];
    }

    // Masked entries get p = 0, but their values may be any bits (rows past a sequence's end in
    // its last block, ring slots never written or stale), and 0 x NaN is NaN: on a tile with
    // such entries their values are zeroed.  V load k holds entry k * TPV + v_tok.
    const uint64_t vis = __ballot(valid);
    if (vis != ~0ull) {
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        if (!((vis >> (k * TPV + v_tok)) & 1ull)) vreg[slot][k] = uint2{0u, 0u};
      }
    }

    // ---- hand p to the PV lanes through the (now free) K stage
    float* pl_lds = reinterpret_cast<float*>(my_k);
#pragma unroll
    for (int pl = 0; pl < GP / 4; ++pl) {
      f32x4 w4;
#pragma unroll
      for (int e = 0; e < 4; ++e) w4[e] = (pl * 4 + e < G) ? p[pl * 4 + e] : 0.f;
      *reinterpret_cast<f32x4*>(pl_lds + (pl * S::TILE + ln) * 4) = w4;
    }

    // ---- PV over this wave's slice of D (fp32 weights, fp32 FMAs)
#pragma unroll
    for (int k = 0; k < NV; ++k) {
      const int tt = k * TPV + v_tok;
      float pp[GP];
#pragma unroll
      for (int pl = 0; pl < GP / 4; ++pl) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(pl_lds + (pl * S::TILE + tt) * 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) pp[pl * 4 + e] = x[e];
      }
      float vf[EV];
      if constexpr (BF16) {
        vf[0] = bf16lo(vreg[slot][k].x);
        vf[1] = bf16hi(vreg[slot][k].x);
        vf[2] = bf16lo(vreg[slot][k].y);
        vf[3] = bf16hi(vreg[slot][k].y);
      } else {
        vf[0] = __uint_as_float(vreg[slot][k].x);
        vf[1] = __uint_as_float(vreg[slot][k].y);
      }
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < EV; ++e) o[g][e] = fmaf(pp[g], vf[e], o[g][e]);
    }
  };

  // One body per tile with a single slot; otherwise three bodies per trip over
  // fixed slots, where leaving early exits the loop, so the latch is only
  // reached after all three and its pending loads always match.
  if (ntiles > 0) {
    if constexpr (kRing == 1) {
      for (int it = 0; it < ntiles; ++it) body(it, 0);
    } else {
#pragma unroll
      for (int i = 0; i < kRing - 1; ++i) issue(i, i, lane);
      __builtin_amdgcn_sched_barrier(0);
      for (int it = 0;; it += kRing) {
        body(it, 0);
        if (it + 1 >= ntiles) break;
        body(it + 1, 1);
        if (it + 2 >= ntiles) break;
        body(it + 2, 2);
        if (it + 3 >= ntiles) break;
      }
    }
  }

  // ---- reduce over the lanes that share a D slot, normalise, write the partial
  float l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = wave_sum(l_lane[g]);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < EV; ++e) o[g][e] = strided_lane_sum<LPR>(o[g][e]);

  const int rows = a.num_q_heads;
  const int pv_tok = lane / LPR, pv_d = lane % LPR;
  float* po = a.part_o + ((int64_t)sg * rows + (int64_t)h * G) * D + wave * (QB / S::ES) + pv_d * EV;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    if (g % TPV == pv_tok) {
      const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
      float* dst = po + (int64_t)g * D;
      if constexpr (EV == 4) {
        const f32x4 w4 = {o[g][0] * inv, o[g][1] * inv, o[g][2] * inv, o[g][3] * inv};
        *reinterpret_cast<f32x4*>(dst) = w4;
      } else {
        const float2 w2 = {o[g][0] * inv, o[g][1] * inv};
        *reinterpret_cast<float2*>(dst) = w2;
      }
    }
  }
  if (wave == 0 && lane < G) {
    float lv = 0.f, mv = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g)
      if (g == lane) { lv = l[g]; mv = M[g]; }
    a.part_lse[(int64_t)sg * rows + (int64_t)h * G + lane] = lv > 0.f ? (mv + __log2f(lv)) * kLn2 : kNegInf;
  }
}

// ----------------------------------------------------------------------------- dispatch
// Window mode (bf16 or fp32 data) and full mode with fp32 data.  Full mode in bf16 runs on the
// whole-tile kernel (wmtp_draft_rows.hip), and bf16 PV weights on the matrix-core kernels.
template <int D, int G, bool BF16>
static hipError_t launch_dg(bool window, const SplitArgs& a, int grid, hipStream_t st) {
  constexpr int T = DraftShape<D, G, BF16>::THREADS;
  if (window) {
    draft_splitk_kernel<D, G, BF16, true><<<grid, T, 0, st>>>(a);
  } else if constexpr (!BF16) {
    draft_splitk_kernel<D, G, BF16, false><<<grid, T, 0, st>>>(a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D, bool BF16>
static hipError_t launch_d(int G, bool window, const SplitArgs& a, int grid, hipStream_t st) {
  switch (G) {
    case 1: return launch_dg<D, 1, BF16>(window, a, grid, st);
    case 2: return launch_dg<D, 2, BF16>(window, a, grid, st);
    case 4: return launch_dg<D, 4, BF16>(window, a, grid, st);
    case 8: return launch_dg<D, 8, BF16>(window, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_draft(int dtype, int head_dim, int group, bool window, const SplitArgs& a, int grid,
                        hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  const bool bf16 = dtype == WMTP_BF16;
  switch (head_dim) {
    case 64: return bf16 ? launch_d<64, true>(group, window, a, grid, st) : launch_d<64, false>(group, window, a, grid, st);
    case 128: return bf16 ? launch_d<128, true>(group, window, a, grid, st) : launch_d<128, false>(group, window, a, grid, st);
    case 256: return bf16 ? launch_d<256, true>(group, window, a, grid, st) : launch_d<256, false>(group, window, a, grid, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace wmtp

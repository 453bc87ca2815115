// Native MTP draft step with fp32 softmax weights on gfx950 vector units: each
// wave owns whole tiles of keys over all of head_dim.
//
// The native draft attends over the whole paged cache at every draft step
// ("Windowed-MTP: Removing the Full-Context Draft-KV Tax at Million-Token
// Context", arxivlens summary, Abstract), so at a million keys it streams the
// 2 GiB layer once per step and must read it at HBM speed.  With fp32 weights
// in the PV product the contraction cannot go through the bf16 matrix cores;
// on the vector units the cost per key is fixed (G x D multiply-adds for QK
// and as many for PV), so what decides the speed is everything around it.
//
// Work item = (sequence b, KV head h, split of `chunk` keys), 8 waves, two per
// SIMD.  Each wave owns whole tiles of 32 keys (16 at d = 256; tiles w, w + 8,
// ... of the split) and keeps its own online-softmax state; nothing is
// exchanged between waves until the end, so the tile loop has no barrier.  The
// G query rows are staged once in LDS.  Per tile and wave:
//   K      coalesced 16-byte non-temporal loads (a wave-load covers one to four
//          rows) into registers one tile ahead; at the top of the tile they go
//          to the wave's own LDS stage, 16-byte pieces XOR-swizzled by row so
//          that "lane = key" reads are free of bank conflicts, and the same
//          registers are reloaded with the next tile.
//   QK     lane = (key, part of D): the lane's part of the row against the G
//          query rows' parts (broadcast LDS reads), bf16 pairs straight into
//          v_dot2_f32_bf16.  The parts are added with lane swaps that each
//          carry two rows, so every lane ends with whole scores of G / parts
//          rows and the softmax runs once per key and row.
//   softmax log2 domain, lazy running maximum per wave (raised and the state
//          rescaled only on a 2^8 jump); the weights go to the wave's LDS slot
//          for the PV lanes.
//   PV     lane = 16-byte slot of a V row (8 values of d), rows as for K, V in
//          registers one tile ahead, each register reloaded once PV has
//          unpacked it; each lane reads the weights of its row's key (a
//          broadcast LDS read) and does G x 8 fp32 FMAs.
// At the end the lanes holding the same d of different rows are summed, the
// waves' states are merged through LDS (the one barrier, after the loop), and
// the split writes its normalised o and lse for the G rows.
#include "wmtp_device.hpp"
#include "wmtp_launch.hpp"

namespace wmtp {

namespace {

constexpr int kRowsWaves = 8;   // waves per work item: two per SIMD

template <int D>
struct RowsShape {
  // Keys per wave tile: 32, or one 16-row block at d = 256, where a 32-key tile of K and V
  // would take 128 registers per lane.
  static constexpr int TK = D == 256 ? 16 : 32;
  static constexpr int ROWB = D * 2;                  // bf16 row bytes
  static constexpr int NPC = ROWB / 16;               // 16-byte pieces per row
  static constexpr int PARTS = 64 / TK;               // QK: lanes per key, each with a part of D
  static constexpr int PPC = NPC / PARTS;             // QK: pieces per part
  static constexpr int RPL = 64 / NPC;                // rows per wave-load (lane = piece of a row)
  static constexpr int LOADS = TK / RPL;              // wave-loads per tile, for K and for V
  static constexpr int NB = TK / kBlock;              // paged blocks per tile
  static constexpr int KSTAGE = TK * ROWB;            // bytes of a wave's K stage
  static_assert(NPC >= 8 && NPC <= 32 && (NPC & (NPC - 1)) == 0, "8..32 pieces per row");
  static_assert(PPC >= 1 && NB >= 1 && RPL <= kBlock, "tile shape");
};

// Physical 16-byte piece of logical piece c of row r in a K stage: 8 consecutive
// rows read by 8 consecutive lanes hit 8 different bank groups.
template <int NPC>
__device__ __forceinline__ int rows_piece(int r, int c) {
  return r * NPC + (c ^ (r & 7));
}

// Sums of lanes l and l ^ 16 (or l ^ 32) for two values at once: the lanes of one parity of
// 16-lane row (of 32-lane half) get a's sum, the others b's.
__device__ __forceinline__ float pack16_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pack32_sum(float a, float b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// x[g] is a lane's partial for row g over its part of D; the PARTS lanes of a key are 16 and 32
// (PARTS 4) or 32 (PARTS 2) apart.  Each lane swap adds two rows' partials at once, so after the
// sums each lane holds the whole scores of G / min(PARTS, G) rows for its key.  Once a single
// value is left, the remaining steps are plain sums (lanes then hold copies).
template <int PARTS, int G>
__device__ __forceinline__ void sum_parts(const float (&x)[G], float (&z)[G / (PARTS < G ? PARTS : G)]) {
  static_assert(PARTS == 2 || PARTS == 4, "2 or 4 lanes per key");
  constexpr int NY = PARTS == 4 ? (G >= 2 ? G / 2 : 1) : G;
  float y[NY];
  if constexpr (PARTS == 4) {
    if constexpr (G >= 2) {
#pragma unroll
      for (int i = 0; i < G / 2; ++i) y[i] = pack16_sum(x[2 * i], x[2 * i + 1]);
    } else {
      y[0] = rows16_sum(x[0]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < G; ++i) y[i] = x[i];
  }
  if constexpr (NY >= 2) {
#pragma unroll
    for (int k = 0; k < NY / 2; ++k) z[k] = pack32_sum(y[2 * k], y[2 * k + 1]);
  } else {
    z[0] = halves_sum(y[0]);
  }
}

// Maximum / sum over the TK lanes of one part (the keys of a tile): a 16-lane row, or a 32-lane
// half.
template <int TK>
__device__ __forceinline__ float key_max(float x) {
  x = fmaxf(x, dpp_f32<kDppXor1>(x));
  x = fmaxf(x, dpp_f32<kDppXor2>(x));
  x = fmaxf(x, dpp_f32<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f32<kDppMirror>(x));
  if constexpr (TK == 32) x = rows16_max(x);
  return x;
}
template <int TK>
__device__ __forceinline__ float key_sum(float x) {
  x += dpp_f32<kDppXor1>(x);
  x += dpp_f32<kDppXor2>(x);
  x += dpp_f32<kDppHalfMirror>(x);
  x += dpp_f32<kDppMirror>(x);
  if constexpr (TK == 32) x = rows16_sum(x);
  return x;
}

}  // namespace

template <int D, int G>
__global__ __launch_bounds__(kRowsWaves * 64, 1) void draft_rows_kernel(const SplitArgs a) {
  using S = RowsShape<D>;
  constexpr int TK = S::TK, ROWB = S::ROWB, NPC = S::NPC, PPC = S::PPC, RPL = S::RPL, LOADS = S::LOADS;
  constexpr int PARTS = S::PARTS;
  constexpr int PE = PARTS < G ? PARTS : G;   // distinct rows per value slot across the parts
  constexpr int NV = G / PE;                  // rows whose scores a lane holds
  constexpr float TAU = 8.0f;   // lazy-max slack, log2 units
  static_assert(G * D * 4 <= S::KSTAGE, "the K stages hold the waves' merge buffers");

  __shared__ __attribute__((aligned(16))) uint8_t k_lds[kRowsWaves * S::KSTAGE];
  __shared__ __attribute__((aligned(16))) uint8_t q_lds[G * ROWB];
  __shared__ __attribute__((aligned(16))) float p_lds[kRowsWaves * TK * G];
  __shared__ float ml_lds[kRowsWaves][2][G];   // per wave: running maximum and normaliser per row
  __shared__ float red_lds[kRowsWaves][G];      // per wave: a tile's maximum per row

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int Hkv = a.num_kv_heads;
  const int h = blockIdx.x % Hkv;
  const int sg = blockIdx.x / Hkv;
  const int b = seq_of_split(a, sg);
  const int n = a.seq_len[b];
  const int t_begin = (sg - a.split_base[b]) * a.chunk;
  const int t_end = min(t_begin + a.chunk, n);
  const int ntiles = (t_end - t_begin + TK - 1) / TK;
  if (a.t_new > 0) append_own_rows<false>(a, b, h, n, max(t_begin, n - a.t_new), t_end, ROWB);

  // the G query rows of this KV head -> LDS (bf16, [G][D])
  {
    const uint8_t* qsrc = static_cast<const uint8_t*>(a.q) + ((int64_t)b * a.num_q_heads + (int64_t)h * G) * ROWB;
    for (int i = threadIdx.x; i < G * NPC; i += blockDim.x)
      *reinterpret_cast<u32x4*>(q_lds + i * 16) = *reinterpret_cast<const u32x4*>(qsrc + i * 16);
  }
  __syncthreads();

  const const_i32_ptr bt_row = as_const_i32(a.block_table) + (int64_t)b * a.bt_stride;
  const int64_t run_bytes = (int64_t)a.run_rows * ROWB;
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k);
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v);
  uint8_t* my_k = k_lds + wave * S::KSTAGE;
  float* my_p = p_lds + wave * (TK * G);

  // This wave's tiles: w, w + 8, ... of the split.
  const int my_tiles = ntiles > wave ? (ntiles - wave + kRowsWaves - 1) / kRowsWaves : 0;
  const int last_blk_idx = (t_end - 1) >> 4;

  // Byte offsets of the (block, head) runs of the blocks of the tile that starts at t0
  // (scalar loads of the table; t0 is wave-uniform and block-aligned, as the split starts at a
  // multiple of 32).  Block indexes past the split's last block are clamped to it, so rows past
  // the split end read valid rows of that block.
  auto tile_runs = [&](int t0, int64_t (&run)[S::NB]) {
#pragma unroll
    for (int jb = 0; jb < S::NB; ++jb) {
      const int bi = min((t0 >> 4) + jb, last_blk_idx);
      run[jb] = paged_block_run(paged_block_uniform(bt_row, (int64_t)bi * kBlock, a.max_block), h, Hkv, run_bytes);
    }
  };

  // Wave-load l covers rows RPL l .. RPL l + RPL - 1 of a tile (one 16-row block: RPL divides
  // 16), lane -> row RPL l + lane / NPC, 16-byte piece lane % NPC.  K and V are read once per
  // launch: non-temporal loads.  One tile of K and one of V are held in registers: a K register
  // is reloaded with the next tile as soon as its rows are in LDS, a V register as soon as PV
  // has used it, so every load has about one tile's work to arrive.
  const uint32_t lane_off = (uint32_t)((lane / NPC) * ROWB + (lane % NPC) * 16);
  u32x4 kreg[LOADS];
  u32x4 vreg[LOADS];
  // The loads for the tile after the wave's last re-read its last one (never consumed).  Each wave
  // reads one tile twice: 1.5% more traffic at a million keys.  Skipping those loads, by peeling
  // the last tile or by a branch, stops the in-place register refill and spills.
  auto tile_of = [&](int it) { return t_begin + (wave + kRowsWaves * min(it, my_tiles - 1)) * TK; };
  auto load_k = [&](const int64_t (&run)[S::NB], int l) __attribute__((always_inline)) {
    const int r0 = RPL * l;
    kreg[l] = load_nt<u32x4>(kbase + run[r0 >> 4] + (r0 & (kBlock - 1)) * ROWB, lane_off);
  };
  auto load_v = [&](const int64_t (&run)[S::NB], int l) __attribute__((always_inline)) {
    const int r0 = RPL * l;
    vreg[l] = load_nt<u32x4>(vbase + run[r0 >> 4] + (r0 & (kBlock - 1)) * ROWB, lane_off);
  };

  const float c = a.scale_log2;
  const int qk_key = lane & (TK - 1);   // QK: key of the lane
  const int qk_part = lane / TK;        // QK: which part of D
  // Byte offset in k_lds of the lane's first K piece: logical piece qk_part PPC + pc of row
  // qk_key is at physical piece ((qk_part PPC) ^ (qk_key & 7)) ^ pc of the row, and rows start
  // at multiples of the row size, so piece pc is at k_x ^ (pc * 16).
  const uint32_t k_x =
      (uint32_t)(wave * S::KSTAGE + qk_key * ROWB + (((qk_part * PPC) ^ (qk_key & 7)) * 16));

  // After the parts are added, value i of a lane is the score of row g_of[i] for key qk_key.
  // Which rows a lane holds follows from the lane swaps: the same additions run once on the row
  // numbers find it (PARTS copies of g add up to PARTS g, exactly).  Lanes of the parts past PE
  // hold copies of rows already held; the "owner" lanes alone count and store weights.
  int g_of[NV];
  {
    float label[G], sum[NV];
#pragma unroll
    for (int g = 0; g < G; ++g) label[g] = (float)g;
    sum_parts<PARTS, G>(label, sum);
#pragma unroll
    for (int i = 0; i < NV; ++i) g_of[i] = (int)(sum[i] * (1.0f / PARTS));
  }
  const bool owner = qk_part < PE;
  int p_slot[NV];   // the lane's weights in the wave's p tile, [key][row]
#pragma unroll
  for (int i = 0; i < NV; ++i) p_slot[i] = qk_key * G + g_of[i];
  float* my_red = red_lds[wave];

  float o[G][8];
  float M[G];              // running maximum of each row (wave-uniform)
  float Mv[NV], l_v[NV];   // the same maxima for the lane's rows; the lane's share of the normalisers
#pragma unroll
  for (int g = 0; g < G; ++g) {
    M[g] = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    Mv[i] = kNegInf;
    l_v[i] = 0.f;
  }

  auto body = [&](int it) __attribute__((always_inline)) {
    const int t0 = t_begin + (wave + kRowsWaves * it) * TK;
    int64_t next_run[S::NB];
    tile_runs(tile_of(it + 1), next_run);
    // ---- K of this tile -> the wave's swizzled LDS stage; the next tile's K into the registers
#pragma unroll
    for (int l = 0; l < LOADS; ++l) {
      *reinterpret_cast<u32x4*>(my_k + rows_piece<NPC>(RPL * l + lane / NPC, lane % NPC) * 16) = kreg[l];
      load_k(next_run, l);
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- QK over the lane's part of D.  The query's LDS address is made opaque per tile so that
    // its reads are not hoisted out of the loop into registers (G x D / PARTS values per lane).
    uint32_t q_off = (uint32_t)(qk_part * PPC * 16);
    asm volatile("" : "+v"(q_off));
    const uint8_t* q_part = q_lds + q_off;
    float acc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) acc[g] = 0.f;
#pragma unroll
    for (int pc = 0; pc < PPC; ++pc) {
      const u32x4 kk = *reinterpret_cast<const u32x4*>(k_lds + (k_x ^ (uint32_t)(pc * 16)));
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const u32x4 qq = *reinterpret_cast<const u32x4*>(q_part + g * ROWB + pc * 16);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[g] = dot2_bf16(qq[e], kk[e], acc[g]);
      }
    }
    // the parts added; each lane keeps the whole scores of NV of the rows
    float s[NV];
    sum_parts<PARTS, G>(acc, s);

    // ---- online softmax (log2 domain, lazy maximum per wave), once per key and row
    const bool valid = t0 + qk_key < t_end;
    bool exceed = false;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      s[i] = valid ? s[i] * c : kNegInf;
      exceed = exceed || (s[i] > Mv[i] + TAU);
    }
    if (__ballot(exceed) != 0) {
      // the tile's maximum of each row: over the lanes that hold it, then gathered for every row
      // through the wave's LDS slot (one lane per row writes; LDS operations of a wave complete
      // in order)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const float tm = key_max<TK>(s[i]);
        const float mn = fmaxf(Mv[i], tm);
        const float alpha = (Mv[i] == kNegInf) ? 0.f : fast_exp2(Mv[i] - mn);
        Mv[i] = mn;
        l_v[i] *= alpha;
        if (qk_key == 0 && owner) my_red[g_of[i]] = tm;
      }
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(M[g], my_red[g]);
        const float alpha = (M[g] == kNegInf) ? 0.f : fast_exp2(M[g] - mn);
        M[g] = mn;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] *= alpha;
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float pi = valid ? fast_exp2(s[i] - Mv[i]) : 0.f;   // s - M <= TAU
      if (owner) {
        l_v[i] += pi;
        my_p[p_slot[i]] = pi;
      }
    }

    // ---- PV: lane = 16-byte slot of a V row.  Rows past the split end carry weight 0, but rows
    // past the sequence's end may hold any bits (0 x NaN is NaN): on the split's last tile,
    // when it is partial, their values are zeroed.
    const int vrow = lane / NPC;
    if (t0 + TK > t_end) {
#pragma unroll
      for (int j = 0; j < LOADS; ++j)
        if (t0 + RPL * j + vrow >= t_end) vreg[j] = u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < LOADS; ++j) {
      const int key = RPL * j + vrow;
      float pw[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int q4 = 0; q4 < G / 4; ++q4) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(my_p + key * G + 4 * q4);
#pragma unroll
          for (int e = 0; e < 4; ++e) pw[4 * q4 + e] = x[e];
        }
      } else {
#pragma unroll
        for (int g = 0; g < G; ++g) pw[g] = my_p[key * G + g];
      }
      const u32x4 vv = vreg[j];
      float vf[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        vf[2 * e] = bf16lo(vv[e]);
        vf[2 * e + 1] = bf16hi(vv[e]);
      }
      // the register is refilled only once its value is unpacked, so the load can land in the
      // same registers (no copy, and no wait for it, at the loop's back edge)
      load_v(next_run, j);
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = fmaf(pw[g], vf[e], o[g][e]);
    }
  };

  if (my_tiles > 0) {
    int64_t run[S::NB];
    tile_runs(tile_of(0), run);
#pragma unroll
    for (int l = 0; l < LOADS; ++l) load_k(run, l);
#pragma unroll
    for (int l = 0; l < LOADS; ++l) load_v(run, l);
    __builtin_amdgcn_sched_barrier(0);
    for (int it = 0; it < my_tiles; ++it) body(it);
  }

  // ---- this wave's state: sum the lanes holding the same d of different rows, and each row's
  // normaliser over its keys
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[g][e] = strided_lane_sum<NPC>(o[g][e]);
  float l_sum[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) l_sum[i] = key_sum<TK>(l_v[i]);
  // ---- merge the waves' states through LDS (the K stages, once every wave is done)
  __syncthreads();
  float* merge = reinterpret_cast<float*>(k_lds);   // [wave][G][D]
  if (lane < NPC) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const f32x4 lo = {o[g][0], o[g][1], o[g][2], o[g][3]};
      const f32x4 hi = {o[g][4], o[g][5], o[g][6], o[g][7]};
      *reinterpret_cast<f32x4*>(merge + (wave * G + g) * D + lane * 8) = lo;
      *reinterpret_cast<f32x4*>(merge + (wave * G + g) * D + lane * 8 + 4) = hi;
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) ml_lds[wave][0][g] = M[g];
  }
  if (qk_key == 0 && owner) {
#pragma unroll
    for (int i = 0; i < NV; ++i) ml_lds[wave][1][g_of[i]] = l_sum[i];
  }
  __syncthreads();
  // rows g = wave, wave + 8, ...: each lane merges D / 64 values of d
  const int rows = a.num_q_heads;
  for (int g = wave; g < G; g += kRowsWaves) {
    float m = kNegInf;
#pragma unroll
    for (int w = 0; w < kRowsWaves; ++w) m = fmaxf(m, ml_lds[w][0][g]);
    float f[kRowsWaves], l = 0.f;
#pragma unroll
    for (int w = 0; w < kRowsWaves; ++w) {
      f[w] = m == kNegInf ? 0.f : fast_exp2(ml_lds[w][0][g] - m);
      l += f[w] * ml_lds[w][1][g];
    }
    const float inv = l > 0.f ? 1.f / l : 0.f;
    const int64_t orow = (int64_t)sg * rows + (int64_t)h * G + g;
    for (int d = lane; d < D; d += 64) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < kRowsWaves; ++w) x = fmaf(f[w], merge[(w * G + g) * D + d], x);
      a.part_o[orow * D + d] = x * inv;
    }
    if (lane == 0) a.part_lse[orow] = l > 0.f ? (m + __log2f(l)) * kLn2 : kNegInf;
  }
}

// ----------------------------------------------------------------------------- dispatch
template <int D>
static hipError_t launch_rows_d(int group, const SplitArgs& a, int grid, hipStream_t st) {
  switch (group) {
    case 1: draft_rows_kernel<D, 1><<<grid, kRowsWaves * 64, 0, st>>>(a); break;
    case 2: draft_rows_kernel<D, 2><<<grid, kRowsWaves * 64, 0, st>>>(a); break;
    case 4: draft_rows_kernel<D, 4><<<grid, kRowsWaves * 64, 0, st>>>(a); break;
    case 8: draft_rows_kernel<D, 8><<<grid, kRowsWaves * 64, 0, st>>>(a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_draft_rows(int head_dim, int group, const SplitArgs& a, int grid, hipStream_t st) {
  if (grid <= 0) return hipSuccess;
  switch (head_dim) {
    case 64: return launch_rows_d<64>(group, a, grid, st);
    case 128: return launch_rows_d<128>(group, a, grid, st);
    case 256: return launch_rows_d<256>(group, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wmtp

// sgmv_fused.h -- gfx950 device code for the fused LoRA delta (included by
// the fused kernel translation units; internal to libsgmv): the LoRA-A
// projection (shrink) and the SGMV expand-slice of its result in one launch,
// with the projected rows kept on chip.
//
// Operation.  The wiki page "Implementation: Predibase Lorax SGMV Expand
// Slice Kernel" describes the expand's inputs as the rank-sized activations
// of the A-side LoRA projection (I/O Contract, Inputs; Usage Examples) and
// motivates the slice kernel by a later operator that fuses several slice
// operations in one launch (Description; Usage: fused QKV and gate/up
// layers).  For segment b with adapter a = idx[b] in [0, lora_num), each row
// t of it and each slice s:
//     y_s[t][k] = rne_w(scale * sum_h x[t][h] * A_s[a][k][h]),    k < K,
//     out[t][off_s + n] = rne_o((add ? out[t][off_s + n] : 0)
//                               + sum_k y_s[t][k] * B_s[a][n][k]),  n < N_s,
// with rne_w the rounding to the 16-bit weight dtype -- exactly what
// sgmv_shrink_multi_slice into weight-dtype outputs followed by
// sgmv_expand_multi_slice computes, without storing y.
//
// Design (MI355X-first).  Two forms, taken by the shrink's own rule so that
// each reproduces one shrink form's sums:
//  * split-T (from shrink_split_t_min_units units of 64 tokens): a work
//    unit is a 64-row tile of one segment.  Phase 1 runs the split-T
//    contraction over the whole hidden dimension (SplitTCore: coalesced
//    input and lora_A loads staged through LDS, MFMAs with lora_A rows as
//    the A operand); phase 2 sweeps every 256-column tile of every slice;
//  * split-H (short prefill and decode batches): a unit is a 16-row tile
//    and a work item is a unit and one column group, about one item per
//    compute unit.  Phase 1 runs the split-H contraction (SplitHCore: the
//    four waves split the hidden steps and add their sums through LDS);
//    phase 2 sweeps the item's column group.
// Phase 1 writes the unit's projected rows, scaled and rounded as the shrink
// stores them, into LDS in the expand's operand layout.  Phase 2
// (FusedExpand) is the expand's: each wave owns 64 columns of a tile, holds
// their lora_B rows in VGPRs, reads the projected rows from LDS as the B
// operand, seeds the accumulators with the prior output (add_inputs) and
// writes the result row-wise through a per-wave LDS tile with non-temporal
// device-scope stores, the next tiles' lora_B rows and prior output loaded
// while the current one computes.  Each accumulator sees the same MFMAs in
// the same order as in the shrink and expand kernels, so the result equals,
// bit for bit, those two calls (shrink without a workspace).
//
// The fused call saves the projection's round trip through memory and a
// launch with its segment table and cold start; it re-reads each adapter's
// lora_B once per unit (16 or 64 rows, from L2), where the expand keeps a
// weight tile for up to 512 rows -- so it pays for small ranks on small
// batches and loses where lora_B is large against a unit's output.
#pragma once

#include "sgmv_device.h"
#include "sgmv_fused_launch.h"
#include "sgmv_shrink.h"

#ifndef SGMV_FUSED_STAGE_REGS
#define SGMV_FUSED_STAGE_REGS 192
#endif

namespace sgmv {
namespace dev {

// Phase 2 of the fused kernels, shared by both forms: the expand of a
// unit's projected rows (kTT token tiles of 16 rows, in LDS) over a range of
// 256-column tiles of the slices.  Each wave owns 64 columns of a tile,
// holds their lora_B rows in VGPRs (the A operand, rows permuted as in the
// expand so that each lane ends with 8 consecutive columns of one token),
// reads the projected rows from LDS as the B operand, seeds the
// accumulators with the prior output (add_inputs) and writes the result
// row-wise through its LDS tile with non-temporal device-scope stores --
// the expand's epilogue; the MFMAs of each accumulator are the expand
// kernel's, in its order.
template <int WD, int OD, bool ADD, int K16, int NS, int kTT>
struct FusedExpand {
  static constexpr int kSteps = K16 >= 2 ? K16 / 2 : 1;  // 32-wide rank steps of the expand
  static constexpr int kKB = 4 * kSteps;                  // 16-byte blocks of a projected row
  static constexpr int kRows = kTileRows * kTT;           // rows of a unit
  static constexpr int ob = OD == F32 ? 4 : 2;
  // Output tile of a wave and token tile (16 rows x 64 columns), accessed
  // row-wise kLPR lanes per row through the per-wave LDS tile, as in the
  // expand (block b of row r in slot kNB r + (b ^ (r mod kNB))).
  static constexpr int kNB = 64 * ob / 16;
  static constexpr int kLPR = kNB;
  static constexpr int kRPI = 64 / kLPR;
  static constexpr int kOAcc = 2 * raw_vecs<OD>();
  static_assert(kOAcc * kRPI == kTileRows, "row-wise accesses cover the tile");
  static_assert(kKB == 4 || kKB == 8 || kKB == 16, "projected row blocks");
  // Ring depth: as many stages (lora_B rows, and the prior output with
  // add_inputs) as about SGMV_FUSED_STAGE_REGS registers hold, 2 to 6.
  static constexpr int kStageRegs = 16 * kSteps + (ADD ? 4 * kTT * kOAcc : 0);
  static constexpr int kRingFit = SGMV_FUSED_STAGE_REGS / kStageRegs;
  static constexpr int kRing = kRingFit < 2 ? 2 : (kRingFit > 6 ? 6 : kRingFit);
  // The unit's projected rows per slice: kRows rows x kKB 16-byte blocks of
  // 16-bit values (rank kept to 32 kSteps, zero past 16 K16).  Block kb of
  // row t in slot t kKB + (kb ^ sw(t)): the operand reads (8 lanes of one
  // g: rows t .. t + 7 at one block) then hit 8 slot classes mod 8.
  typedef u32x4 YLds[NS][kRows * kKB];
  typedef u32x4 OLds[kWaves][kTileRows * kNB];
  __device__ __forceinline__ static int y_slot(int t, int kb) {
    const int sw = kKB >= 8 ? (t & 7) : ((t >> 1) & 3);
    return t * kKB + (kb ^ sw);
  }
  __device__ __forceinline__ static int o_slot(int r, int b) { return kNB * r + (b ^ (r % kNB)); }

  // One column tile as this wave sees it.
  struct Tile {
    rsrc_t w;            // lora_B rows [col0, col0 + n_rem) of the unit's adapter
    uint32_t col_bytes;  // byte offset of column off_s + col0 within a row
    int32_t n_rem;       // columns of the wave (<= 0: none)
    int si;              // slice
  };
  struct Stage {
    u32x4 w[4][kSteps];
    u32x4 o[ADD ? kTT : 1][ADD ? kOAcc : 1];
  };

  YLds& y_lds;
  OLds& o_lds;
  int lane, wave, g, j, orow, oblk, ocol, K;
  uint32_t o_row_off[kTT][kOAcc];

  __device__ __forceinline__ FusedExpand(const FusedParams& p, YLds& y, OLds& o)
      : y_lds(y), o_lds(o) {
    lane = threadIdx.x & 63;
    wave = uniform(threadIdx.x >> 6);
    g = lane >> 4;
    j = lane & 15;
    K = p.K;
    // this lane's block of a row-wise access and its byte offsets within the
    // unit's rows
    orow = lane / kLPR;
    oblk = lane % kLPR;
    ocol = oblk * (16 / ob);
    const uint32_t orb = (uint32_t)p.out_row_bytes;  // 64 rows span < 2 GiB (host)
#pragma unroll
    for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
      for (int m = 0; m < kOAcc; ++m)
        o_row_off[tt][m] =
            (uint32_t)(kTileRows * tt + m * kRPI + orow) * orb + (uint32_t)(oblk * 16);
  }

  // Rank 16 and below: the expand's rank step also reads k 16 .. 31, which
  // the projection never writes; they stay zero (ordered before the first
  // read by the barriers of the first unit's projection).
  __device__ __forceinline__ void clear_rank_tail() {
    if constexpr (16 * K16 < 32 * kSteps) {
      for (int i = threadIdx.x; i < NS * kRows; i += kThreads) {
        const int s = i / kRows, t = i % kRows;
        for (int kb = 2 * K16; kb < kKB; ++kb) y_lds[s][y_slot(t, kb)] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // Lane (j, g) of k tile kt of slice si holds the scaled sums of k = 16 kt +
  // 4 g .. + 3 of row t: rounded to the weight dtype into y_lds.
  __device__ __forceinline__ void put(int si, int kt, int t, f32x4 v) {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    u32x2* dst = reinterpret_cast<u32x2*>(&y_lds[si][y_slot(t, 2 * kt + (g >> 1))]) + (g & 1);
    *dst = u32x2{pack2<WD>(v[0], v[1]), pack2<WD>(v[2], v[3])};
  }

  // Column tiles [ct_lo, ct_hi) of rows [row0, row0 + rows) with adapter a.
  __device__ __forceinline__ void run(const FusedParams& p, int32_t row0, int32_t rows, int64_t a,
                                      int32_t ct_lo, int32_t ct_hi) {
    const rsrc_t orc = make_rsrc(static_cast<char*>(p.out) + (int64_t)row0 * p.out_row_bytes,
                                 (int64_t)rows * p.out_row_bytes);
    auto w_off = [&](int s, int ks) __attribute__((always_inline)) -> uint32_t {
      const int kb = 32 * ks + 8 * g;
      return kb < K ? (uint32_t)((weight_row(0, s, j) * K + kb) * 2) : kOut;
    };
    auto acc_blk = [&](int q, int v) __attribute__((always_inline)) -> int {
      return raw_vecs<OD>() == 1 ? 4 * q + g : 2 * (4 * q + g) + v;
    };
    auto tile_at = [&](int ct) __attribute__((always_inline)) -> Tile {
      int si = 0;
#pragma unroll
      for (int s = 1; s < NS; ++s)
        if (ct >= p.s[s].tile_begin) si = s;
      const FusedSliceDesc& S = p.s[si];
      const int32_t col0 = (ct - S.tile_begin) * kTileCols + wave * kWaveCols;
      const int64_t left = ct < ct_hi ? S.n - col0 : 0;
      Tile tl;
      tl.si = si;
      tl.n_rem = left <= 0 ? 0 : (left > kWaveCols ? kWaveCols : (int32_t)left);
      tl.col_bytes = (uint32_t)((S.offset + col0) * ob);
      tl.w = make_rsrc(static_cast<const char*>(S.w) + (a * S.n + col0) * K * 2,
                       (int64_t)tl.n_rem * K * 2);
      return tl;
    };
    auto load_stage = [&](Stage& st, const Tile& tl) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) buf_load8<WD>(tl.w, w_off(s, ks), &st.w[s][ks]);
      if constexpr (ADD) {
#pragma unroll
        for (int tt = 0; tt < kTT; ++tt)
#pragma unroll
          for (int m = 0; m < kOAcc; ++m)
            st.o[tt][m] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           orc, ocol < tl.n_rem ? o_row_off[tt][m] + tl.col_bytes : kOut, 0, 0));
      }
    };
    auto compute_store = [&](const Stage& st, const Tile& tl) __attribute__((always_inline)) {
#pragma unroll
      for (int tt = 0; tt < kTT; ++tt) {
        f32x4 acc[4];
        if constexpr (ADD) {
          // row-wise prior output -> the wave's LDS tile -> accumulator layout
#pragma unroll
          for (int m = 0; m < kOAcc; ++m) o_lds[wave][o_slot(m * kRPI + orow, oblk)] = st.o[tt][m];
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
          if constexpr (ADD) {
            u32x4 raw[raw_vecs<OD>()];
#pragma unroll
            for (int rv = 0; rv < raw_vecs<OD>(); ++rv)
              raw[rv] = o_lds[wave][o_slot(j, acc_blk(q, rv))];
            out_values<OD>(raw, v);
          }
          acc[2 * q] = f32x4{v[0], v[1], v[2], v[3]};
          acc[2 * q + 1] = f32x4{v[4], v[5], v[6], v[7]};
        }
#pragma unroll
        for (int ks = 0; ks < kSteps; ++ks) {
          const u32x4 yo = y_lds[tl.si][y_slot(kTileRows * tt + j, 4 * ks + g)];
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[s] = mfma<WD>(st.w[s][ks], yo, acc[s]);
        }
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const float v[8] = {acc[2 * q][0], acc[2 * q][1], acc[2 * q][2], acc[2 * q][3],
                              acc[2 * q + 1][0], acc[2 * q + 1][1], acc[2 * q + 1][2],
                              acc[2 * q + 1][3]};
          u32x4 raw[raw_vecs<OD>()];
          out_pack<OD>(v, raw);
#pragma unroll
          for (int rv = 0; rv < raw_vecs<OD>(); ++rv)
            o_lds[wave][o_slot(j, acc_blk(q, rv))] = raw[rv];
        }
        // rows past the unit's tokens lie outside orc; columns past the
        // slice take the out-of-range offset
#pragma unroll
        for (int m = 0; m < kOAcc; ++m)
          __builtin_amdgcn_raw_buffer_store_b128(
              o_lds[wave][o_slot(m * kRPI + orow, oblk)], orc,
              ocol < tl.n_rem ? o_row_off[tt][m] + tl.col_bytes : kOut, 0, kStream);
      }
    };

    // A ring of kRing stages: the loads of column tile c + kRing - 1 are
    // issued before tile c computes and stores.  On gfx9 the vector-memory
    // counter covers stores as well as loads and retires in issue order, so
    // waiting for a tile's loads also waits for every store issued before
    // them: with the loads kRing - 1 tiles ahead, a tile's stores have
    // kRing - 1 tiles of work to complete before anything waits on them
    // (with one tile ahead, every tile paid a store round trip: fused
    // gate/up 3.7 us per tile).  The loop runs over whole turns of the
    // ring; positions past the last tile load nothing and store nothing.
    Stage ring[kRing];
    Tile tr[kRing];
#pragma unroll
    for (int d = 0; d + 1 < kRing; ++d) {
      tr[d] = tile_at(ct_lo + d);
      load_stage(ring[d], tr[d]);
    }
    for (int ct = ct_lo; ct < ct_hi; ct += kRing) {
#pragma unroll
      for (int d = 0; d < kRing; ++d) {
        const int nxt = (d + kRing - 1) % kRing;
        tr[nxt] = tile_at(ct + d + kRing - 1);
        load_stage(ring[nxt], tr[nxt]);
        __builtin_amdgcn_sched_barrier(0);
        compute_store(ring[d], tr[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

// Large batches: a unit is a 64-row tile of one segment (the split-T
// shrink's unit); phase 1 is the split-T contraction, phase 2 sweeps every
// column tile of every slice.
template <int XD, int WD, int OD, bool ADD, int K16, int NS>
__global__ __launch_bounds__(kThreads) void fused_shrink_expand(const FusedParams p) {
  using Core = SplitTCore<XD, WD, K16, NS>;
  using Exp = FusedExpand<WD, OD, ADD, K16, NS, kFusedTokens / kTileRows>;
  prefetch_params(p);
  extern __shared__ __align__(16) int32_t lds[];  // segment table, 4 * batches + 1 words
  __shared__ int32_t wave_total[kWaves];
  __shared__ typename Core::ALds a_lds;
  __shared__ typename Core::XLds x_lds;
  __shared__ typename Exp::YLds y_lds;
  __shared__ typename Exp::OLds o_lds;
  const SegTable tab = seg_table(lds, p.batches);
  const int32_t U = build_tile_table(p, tab, wave_total, kFusedTokens);
  if (U == 0) return;
  uint32_t u, u_end;
  unit_range(p, (uint32_t)U, &u, &u_end);
  if (u >= u_end) return;

  Core core(p, a_lds, x_lds);
  Exp ex(p, y_lds, o_lds);
  ex.clear_rank_tail();
  int b = last_at_most(tab.tile_start, p.batches + 1, (int32_t)u);
  for (; u < u_end; ++u) {
    while (uniform(tab.tile_start[b + 1]) <= (int32_t)u) ++b;
    const ShrinkUnit<NS> su = shrink_unit<NS>(p, tab, b, u, kFusedTokens);
    const int64_t a = uniform(tab.seg_lora[b]);

    // Phase 1: the unit's projection, scaled and rounded to the weight
    // dtype as the shrink stores it, into y_lds.  The barrier first orders
    // the previous unit's reads of y_lds before these writes.
    {
      f32x4 acc[Core::kTok][Core::kKt];
      core.run(su, acc, 0, p.steps);
      __syncthreads();
#pragma unroll
      for (int h = 0; h < Core::kTok; ++h)
#pragma unroll
        for (int i = 0; i < Core::kKt; ++i) {
          const int kg = core.k_tile(i);
          ex.put(kg / K16, kg % K16, kTileRows * core.tok_tile(h) + core.j, acc[h][i] * p.scale);
        }
      __syncthreads();
    }
    // Phase 2: every column tile of every slice.
    ex.run(p, su.row0, su.rows, a, 0, p.total_tiles);
  }
}

// Small batches: a unit is a 16-row tile of one segment (the split-H
// shrink's unit) and a work item is a unit and one of G column groups
// (contiguous ranges of the 256-column tiles; G from p.item_target and the
// unit count), so that a batch of few units still spreads its expansion
// over the chip.  Phase 1 is the split-H contraction (each item of a unit
// computes it); phase 2 sweeps the item's column group.  Items of one unit
// are adjacent, so they run on one XCD and share its L2 for the unit's
// inputs and lora_A rows.
template <int XD, int WD, int OD, bool ADD, int K16, int NS>
__global__ __launch_bounds__(kThreads) void fused_split_h(const FusedParams p) {
  using Core = SplitHCore<XD, WD, K16, NS>;
  using Exp = FusedExpand<WD, OD, ADD, K16, NS, 1>;
  prefetch_params(p);
  extern __shared__ __align__(16) int32_t lds[];  // segment table, 4 * batches + 1 words
  __shared__ int32_t wave_total[kWaves];
  __shared__ typename Core::RedLds red;
  __shared__ typename Core::StageLds stage;
  __shared__ typename Exp::YLds y_lds;
  __shared__ typename Exp::OLds o_lds;
  const SegTable tab = seg_table(lds, p.batches);
  const int32_t U = build_tile_table(p, tab, wave_total, kTileRows);
  if (U == 0) return;
  // Column groups per unit: as many as bring the items up to the target,
  // at most one per column tile.
  const uint32_t tgt = (uint32_t)p.item_target, UU = (uint32_t)U;
  uint32_t G = tgt > UU ? tgt / UU : 1u;
  if (G > (uint32_t)p.total_tiles) G = (uint32_t)p.total_tiles;
  uint32_t it, it_end;
  unit_range(p, (uint32_t)U * G, &it, &it_end);
  if (it >= it_end) return;

  Core core(p, red, stage);
  Exp ex(p, y_lds, o_lds);
  ex.clear_rank_tail();
  const int32_t tiles = p.total_tiles;
  int b = last_at_most(tab.tile_start, p.batches + 1, (int32_t)(it / G));
  for (; it < it_end; ++it) {
    const uint32_t u = it / G, cg = it % G;
    while (uniform(tab.tile_start[b + 1]) <= (int32_t)u) ++b;
    const ShrinkUnit<NS> su = shrink_unit<NS>(p, tab, b, u, kTileRows);
    // Phase 1: the four waves' partial sums added in wave order (the
    // reduction's first barrier orders the previous item's reads of y_lds
    // before these writes), scaled and rounded into y_lds.  With several
    // column groups per unit every workgroup has one item (the host caps
    // p.item_target at the grid), so no projection is ever recomputed on one
    // workgroup.
    {
      f32x4 acc[Core::kT];
      core.run(su, acc, p.steps);
      core.reduce(acc, [&](int i, f32x4 v) __attribute__((always_inline)) {
        ex.put(i / K16, i % K16, core.j, v * p.scale);
      });
      __syncthreads();
    }
    // Phase 2: column tiles [cg tiles / G, (cg + 1) tiles / G).
    const int32_t lo = (int32_t)(((int64_t)cg * tiles) / G);
    const int32_t hi = (int32_t)(((int64_t)(cg + 1) * tiles) / G);
    ex.run(p, su.row0, su.rows, uniform(tab.seg_lora[b]), lo, hi);
  }
}

// ---------------------------------------------------------------------------
// Kernel tables.
// ---------------------------------------------------------------------------

template <int XD, int WD, int OD, int K16>
const void* fused_by_ns(bool add, int ns, bool split_h) {
  auto pick = [&](auto nsc) -> const void* {
    constexpr int NS = decltype(nsc)::value;
    if constexpr (K16 * NS > 16) {
      return nullptr;
    } else if (split_h) {
      return add ? reinterpret_cast<const void*>(&fused_split_h<XD, WD, OD, true, K16, NS>)
                 : reinterpret_cast<const void*>(&fused_split_h<XD, WD, OD, false, K16, NS>);
    } else {
      return add ? reinterpret_cast<const void*>(&fused_shrink_expand<XD, WD, OD, true, K16, NS>)
                 : reinterpret_cast<const void*>(&fused_shrink_expand<XD, WD, OD, false, K16, NS>);
    }
  };
  switch (ns) {
    case 1: return pick(std::integral_constant<int, 1>{});
    case 2: return pick(std::integral_constant<int, 2>{});
    case 3: return pick(std::integral_constant<int, 3>{});
    default: return nullptr;
  }
}

template <int XD, int WD, int K16>
const void* fused_by_out(int od, bool add, int ns, bool split_h) {
  switch (od) {
    case F16: return fused_by_ns<XD, WD, F16, K16>(add, ns, split_h);
    case BF16: return fused_by_ns<XD, WD, BF16, K16>(add, ns, split_h);
    case F32: return fused_by_ns<XD, WD, F32, K16>(add, ns, split_h);
    default: return nullptr;
  }
}

template <int K16>
const void* fused_table(int xd, int wd, int od, bool add, int ns, bool split_h) {
  if (wd == BF16 && xd == BF16) return fused_by_out<BF16, BF16, K16>(od, add, ns, split_h);
  if (wd == BF16 && xd == F32) return fused_by_out<F32, BF16, K16>(od, add, ns, split_h);
  if (wd == F16 && xd == F16) return fused_by_out<F16, F16, K16>(od, add, ns, split_h);
  if (wd == F16 && xd == F32) return fused_by_out<F32, F16, K16>(od, add, ns, split_h);
  return nullptr;
}

}  // namespace dev
}  // namespace sgmv

// sgmv_shrink.h -- gfx950 device code for the LoRA-A projection (shrink),
// the step that produces SGMV expand-slice's inputs (included by the shrink
// kernel translation units; internal to libsgmv).
//
// Operation: the wiki page "Implementation: Predibase Lorax SGMV Expand
// Slice Kernel" (I/O Contract, Inputs; Usage Examples) describes the
// expand's inputs as the rank-sized activations the A-side LoRA projection
// produces for every token of every sequence, (total_tokens, rank).  For
// segment b with adapter a = idx[b] in [0, lora_num) and each row t of it,
//     y_s[t][k] = scale * sum_h x[t][h] * A_s[a][k][h],   k in [0, K),
// for every slice s (lora_A stack A_s (L, K, H), output y_s (T, K)).  Rows of
// other segments are not written.  float32 inputs are rounded to the weight
// dtype first, as in the expand.
//
// Design.  The projection reads every input row once and writes a row of K
// values, so it is bound by reading x (and, with many adapters and short
// segments, by reading the lora_A stacks).  The slices share the input tile:
// their lora_A rows are just more K rows (k tiles) of one contraction, so a
// fused QKV projection reads x once.  Two kernel forms:
//  * split-H: a work unit is a 16-row tile of one segment; the four
//    wavefronts split the hidden dimension, each streams its part of the 16
//    input rows and of every lora_A row the slices need, and the partial
//    sums are added through LDS at the end of the unit;
//  * split-T (enough tokens): a unit is a 64-row tile, every wave runs the
//    whole hidden dimension, and the lora_A blocks are loaded once per
//    workgroup and shared through LDS; wave t owns tokens 16 t .. 16 t + 15,
//    or, with an even number of k tiles (at least 4), 32 tokens and half of
//    the k tiles, so that each fragment read from LDS feeds two MFMAs.
//    With a caller's workspace and between C and 2 C units (C compute
//    units), the units past the first C are cut into parts over the hidden
//    steps that run beside the whole units, so that no compute unit runs
//    two whole units while others run one; with at most C / 2 units, every
//    unit is cut into parts, so that the idle compute units share the work.
//    The last part of each unit adds the parts' fp32 sums in part order
//    (limits::part_plan, reduce_parts).
//
// The contraction is y^T = A . x^T on the matrix cores
// (v_mfma_f32_16x16x32_{bf16,f16}): 16 lora_A rows are the A operand, the 16
// tokens of the tile the B operand, 32 hidden elements per instruction; each
// lane ends with 4 consecutive k of one token per k tile.  Loads are
// coalesced -- 128 or more contiguous bytes of each row per instruction --
// and staged through LDS into the MFMA operand order.  Input rows are read
// once, so their loads are non-temporal (measured on MI355X, streaming reads
// are markedly faster that way); lora_A rows are re-read by the units of an
// adapter and keep the default policy.  Loads go through buffer resources
// bounded by the tile's valid rows and the slice's K rows, so rows past the
// segment and k past K read zero and store nothing; hidden blocks past H
// take an offset outside every resource.  The step loop runs over a ring of
// blocks in registers, issuing each block several blocks ahead of its use;
// every block issues the same load instructions (blocks past the end read
// nothing), so the compiler waits for one block with a nonzero vmcnt.
#pragma once

#include "sgmv_common.h"
#include "sgmv_shrink_launch.h"

namespace sgmv {
namespace dev {

// Four consecutive outputs at byte offset `off` of resource r.
template <int OD>
__device__ __forceinline__ void store4(rsrc_t r, uint32_t off, f32x4 v) {
  if constexpr (OD == F32) {
    __builtin_amdgcn_raw_buffer_store_b128(
        u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
              __float_as_uint(v[3])},
        r, (int)off, 0, 0);
  } else {
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    __builtin_amdgcn_raw_buffer_store_b64(u32x2{pack2<OD>(v[0], v[1]), pack2<OD>(v[2], v[3])},
                                          r, (int)off, 0, 0);
  }
}

// Compile-time shape: K16 16-row k tiles per slice, NS slices; k tile i of
// the launch is tile i % K16 of slice i / K16.
template <int XD, int K16, int NS>
struct ShrinkShape {
  static constexpr int kTiles = K16 * NS;
  static constexpr int kNV = raw_vecs<XD>();
  static constexpr int kBlockH = shrink_block_steps_h(XD, kTiles);
  static constexpr int kBlockT = shrink_block_steps_t(kTiles);
  // split-T: lora_A loads of one slice's block that each wave issues (one
  // load = 8 rows x 128 bytes, i.e. half a k tile over two steps)
  static constexpr int kPairs = K16 * kBlockT / kWaves;
  // blocks in flight
  static constexpr int kRingH = shrink_ring(shrink_block_loads_h(XD, kTiles));
  static constexpr int kRingT = shrink_ring(shrink_block_loads_t(XD, K16, NS));
  static_assert(kTiles <= 16 && NS <= kShrinkMaxSlicesPerLaunch, "shape");
  static_assert(K16 * kBlockT % kWaves == 0, "split-T loads divide among the waves");
  static_assert(kBlockT % 2 == 0, "split-T lora_A loads cover two steps");
};

// One unit as the kernels see it: first row, valid rows, adapter, and the
// resources over the unit's input rows and each slice's lora_A[a].
template <int NS>
struct ShrinkUnit {
  int32_t row0, rows;
  rsrc_t x;
  rsrc_t a[NS];
};

template <int NS, typename P>
__device__ __forceinline__ ShrinkUnit<NS> shrink_unit(const P& p, const SegTable& tab,
                                                      int b, uint32_t u, int32_t tile_rows) {
  ShrinkUnit<NS> su;
  su.row0 = uniform(tab.seg_row[b]) + ((int32_t)u - uniform(tab.tile_start[b])) * tile_rows;
  const int32_t left = uniform(tab.seg_end[b]) - su.row0;
  su.rows = left < tile_rows ? left : tile_rows;
  const int64_t a = uniform(tab.seg_lora[b]);
  su.x = make_rsrc(static_cast<const char*>(p.x) + (int64_t)su.row0 * p.x_row_bytes,
                   (int64_t)su.rows * p.x_row_bytes);
  const int64_t a_bytes = (int64_t)p.K * p.H * 2;  // one adapter's (K, H) block
#pragma unroll
  for (int s = 0; s < NS; ++s)
    su.a[s] = make_rsrc(static_cast<const char*>(p.s[s].a) + a * a_bytes, a_bytes);
  return su;
}

// Store a wave's 16 x 16 fragment i (k tile i % K16 of slice i / K16) of the
// token tile starting `trow` rows into the unit: lane (j, g) holds k = 16 kt +
// 4 g .. + 3 of token trow + j.
template <int OD, int K16>
__device__ __forceinline__ void shrink_store(const ShrinkParams& p, int i, int32_t row0,
                                             int32_t rows, int trow, int j, int g, f32x4 v) {
  constexpr int ob = OD == F32 ? 4 : 2;
  const int si = i / K16, kt = i % K16;
  const ShrinkSliceDesc& S = p.s[si];
  const rsrc_t orc = make_rsrc(static_cast<char*>(S.out) + (int64_t)row0 * S.out_row_bytes,
                               (int64_t)rows * S.out_row_bytes);
  const int32_t k = 16 * kt + 4 * g;
  const uint32_t off =
      k < p.K ? (uint32_t)(trow + j) * (uint32_t)S.out_row_bytes + (uint32_t)(k * ob) : kOut;
  store4<OD>(orc, off, v * p.scale);
}

// LDS layout of an operand fragment staged from coalesced loads (16 rows x
// 32 hidden, 1 KiB in MFMA operand order, lora_A or input), both kernels:
// lane (j, g)'s 16 bytes sit in slot 16 g + (j ^ 2 g) of the fragment, and
// fragments are kFragSlots = 65 slots apart.  The LDS serves a 16-byte
// access 8 lanes (128 bytes, 8 slot classes mod 8) at a time (measured on
// gfx950 with the SQ_LDS_BANK_CONFLICT counter).  The MFMA operand reads
// (8 lanes of one g, consecutive j) hit 8 classes for any g.  The staging
// writes of a coalesced load put 8 lanes on one row: g = 0..3 of two
// consecutive steps, i.e. of fragments f and f + 1; they hit the 4 classes
// of one parity in fragment f and, 65 being odd, the other 4 in f + 1.
// (Slot 16 g + (j ^ 4 g) hits 4 classes there: 2-way conflicts.)
constexpr int kFragSlots = 65;
__device__ __forceinline__ int frag_slot(int j, int g) { return 16 * g + (j ^ (2 * g)); }

// ---------------------------------------------------------------------------
// Split-H: 16 tokens per unit; the four waves of the workgroup split the
// hidden steps and add their partial sums through LDS.
// ---------------------------------------------------------------------------

template <int XD, int K16, int NS>
struct SplitHBlock {
  using Sh = ShrinkShape<XD, K16, NS>;
  u32x4 x[Sh::kBlockH][Sh::kNV];
  u32x4 a[Sh::kBlockH][Sh::kTiles];
};

// The split-H contraction of one 16-token unit, shared by the shrink kernel
// and the fused shrink-expand kernel for small batches: `run` leaves in
// acc[i] this wave's fp32 partial sums over its quarter of the hidden steps
// (k tile i of the launch is tile i % K16 of slice i / K16); `reduce` adds
// the four waves' partial sums through LDS in wave order and hands each
// finished fragment to emit(i, v), lane (j, g) holding k = 16 (i % K16) +
// 4 g .. + 3 of token j.  The LDS buffers are the caller's (declared in the
// kernel).  P: a parameter block with the ShrinkParams fields x_row_bytes,
// H and s[].a.
template <int XD, int WD, int K16, int NS>
struct SplitHCore {
  using Sh = ShrinkShape<XD, K16, NS>;
  using Block = SplitHBlock<XD, K16, NS>;
  static constexpr int kW = kWaves;
  static constexpr int kT = Sh::kTiles;
  static constexpr int kB = Sh::kBlockH;
  // fragments added per LDS round: kW x kRound fragments of 1 KiB <= 32 KiB
  static constexpr int kRound = kT < 32 / kW ? kT : 32 / kW;
  static constexpr int xb = XD == F32 ? 4 : 2;
  // Coalesced loads (up to 8 k tiles): load i of a block reads rows
  // i kRPI .. + kRPI - 1 of a 16-row tile, kLPR lanes per row covering the
  // block's kB steps contiguously (lane l: row l / kLPR, hidden block
  // l % kLPR, i.e. block (l % kLPR) % 4 of step (l % kLPR) / 4); the wave
  // scatters them into MFMA operand order in its own LDS region (see
  // frag_slot) and reads the operands back.  More k tiles load operands
  // directly (16 rows x 64 bytes per load), which needs no LDS.
  static constexpr bool kCoal = kT <= 8;
  static constexpr int kLPR = 4 * kB;
  static constexpr int kRPI = 64 / kLPR;
  static_assert(!kCoal || (kB % 2 == 0 && kRPI * kB == 16), "coalesced block shape");
  typedef f32x4 RedLds[kW][kRound][64];
  // per wave: the block's input fragments (steps 0 .. kB - 1), then each k
  // tile's ([tile + 1] kB + step)
  typedef u32x4 StageLds[kCoal ? kW : 1][kCoal ? (kT + 1) * kB : 1][kCoal ? kFragSlots : 1];

  RedLds& red;
  StageLds& stage;
  int lane, wave, g, j, cr, cb, cst, cg, r_slot;
  int32_t H, q_steps, s_beg;
  uint32_t xrb, x_lane, xc_lane, ac_lane;
  uint32_t a_lane[K16];  // row 16 kt + j of a slice's lora_A[a], hidden block 8 g

  template <typename P>
  __device__ __forceinline__ SplitHCore(const P& p, RedLds& r, StageLds& s) : red(r), stage(s) {
    lane = threadIdx.x & 63;
    wave = uniform(threadIdx.x >> 6);
    g = lane >> 4;  // lane group: hidden block 8 g of a step / k rows 4 g.. of a tile
    j = lane & 15;  // token of the tile / lora_A row of a k tile
    H = p.H;
    xrb = (uint32_t)p.x_row_bytes;  // 16 rows span < 2 GiB (host)
    // The wave's hidden steps: [wave q, wave q + q) with q = ceil(steps / kW),
    // run over p.steps >= q loop positions (the rest read nothing).
    q_steps = (((H + 31) >> 5) + kW - 1) / kW;
    s_beg = wave * q_steps;
    // direct operand loads: row j, hidden block 8 g
    x_lane = (uint32_t)j * xrb + (uint32_t)(8 * g * xb);
#pragma unroll
    for (int kt = 0; kt < K16; ++kt)
      a_lane[kt] = (uint32_t)(16 * kt + j) * (uint32_t)H * 2u + (uint32_t)(16 * g);
    // coalesced loads: row cr of the load, hidden block cb of the block's span
    cr = lane / kLPR;
    cb = lane % kLPR;
    cst = cb >> 2;  // its step within the block and block in the step
    cg = cb & 3;
    xc_lane = (uint32_t)cr * xrb + (uint32_t)(8 * cb * xb);
    ac_lane = (uint32_t)cr * (uint32_t)H * 2u + (uint32_t)(16 * cb);
    r_slot = frag_slot(j, g);
  }

  // The wave's partial sums of unit su over its hidden steps; `steps` loop
  // positions (a multiple of the ring's turn).
  __device__ __forceinline__ void run(const ShrinkUnit<NS>& su, f32x4 (&acc)[kT], int32_t steps) {
    // the lane constants as locals of the loop (members captured through
    // `this` cost registers in the ring loop)
    const int32_t H = this->H, q_steps = this->q_steps, s_beg = this->s_beg;
    const uint32_t xrb = this->xrb, x_lane = this->x_lane, xc_lane = this->xc_lane,
                   ac_lane = this->ac_lane;
    const int wave = this->wave, g = this->g, cr = this->cr, cst = this->cst, cg = this->cg,
              r_slot = this->r_slot;
    uint32_t a_lane[K16];
#pragma unroll
    for (int kt = 0; kt < K16; ++kt) a_lane[kt] = this->a_lane[kt];
    StageLds& stage = this->stage;
    auto load_block = [&](Block& blk, int32_t v0) __attribute__((always_inline)) {
      if constexpr (kCoal) {
        const int32_t v = v0 + cst;  // this lane's step
        const int32_t step = s_beg + v;
        const bool ok = v < q_steps && 32 * step + 8 * cg < H;
        const uint32_t span = (uint32_t)(s_beg + v0);  // the block's first step
#pragma unroll
        for (int i = 0; i < kB; ++i) {
          const uint32_t rows = (uint32_t)(i * kRPI);
          buf_load8<XD, kStreamLoad>(su.x, ok ? xc_lane + rows * xrb + span * (uint32_t)(32 * xb) : kOut,
                        blk.x[i]);
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int kt = 0; kt < K16; ++kt)
              buf_load8<WD>(su.a[s],
                            ok ? ac_lane + (16u * kt + rows) * (uint32_t)H * 2u + span * 64u : kOut,
                            &blk.a[i][s * K16 + kt]);
        }
      } else {
#pragma unroll
        for (int st = 0; st < kB; ++st) {
          const int32_t v = v0 + st;
          const int32_t step = s_beg + v;
          const bool ok = v < q_steps && 32 * step + 8 * g < H;
          buf_load8<XD, kStreamLoad>(su.x, ok ? x_lane + (uint32_t)(32 * step * xb) : kOut, blk.x[st]);
#pragma unroll
          for (int s = 0; s < NS; ++s)
#pragma unroll
            for (int kt = 0; kt < K16; ++kt)
              buf_load8<WD>(su.a[s], ok ? a_lane[kt] + (uint32_t)(64 * step) : kOut,
                            &blk.a[st][s * K16 + kt]);
        }
      }
    };
#pragma unroll
    for (int i = 0; i < kT; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute_block = [&](const Block& blk) __attribute__((always_inline)) {
      if constexpr (kCoal) {
        // scatter into operand order (float32 inputs rounded to the weight
        // dtype here), then read the operands back; one wave's region, so
        // the LDS keeps the writes and reads in order without a barrier
#pragma unroll
        for (int i = 0; i < kB; ++i) {
          const int sl = frag_slot(i * kRPI + cr, cg);
          stage[wave][cst][sl] = x_operand<XD, WD>(blk.x[i]);
#pragma unroll
          for (int t = 0; t < kT; ++t) stage[wave][(t + 1) * kB + cst][sl] = blk.a[i][t];
        }
#pragma unroll
        for (int st = 0; st < kB; ++st) {
          const u32x4 xo = stage[wave][st][r_slot];
#pragma unroll
          for (int t = 0; t < kT; ++t)
            acc[t] = mfma<WD>(stage[wave][(t + 1) * kB + st][r_slot], xo, acc[t]);
        }
      } else {
#pragma unroll
        for (int st = 0; st < kB; ++st) {
          const u32x4 xo = x_operand<XD, WD>(blk.x[st]);
#pragma unroll
          for (int i = 0; i < kT; ++i) acc[i] = mfma<WD>(blk.a[st][i], xo, acc[i]);
        }
      }
    };

    // Loop positions [0, steps) (a multiple of kD kB): a ring of kD blocks
    // in registers, block n + kD - 1 issued before block n computes.
    // Scheduling barriers keep each block's loads in issue order, which the
    // in-order vmcnt wait relies on.
    constexpr int kD = Sh::kRingH;
    Block ring[kD];
#pragma unroll
    for (int d = 0; d + 1 < kD; ++d) {
      load_block(ring[d], d * kB);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int32_t s = 0; s < steps; s += kD * kB) {
#pragma unroll
      for (int d = 0; d < kD; ++d) {
        load_block(ring[(d + kD - 1) % kD], s + (d + kD - 1) * kB);
        __builtin_amdgcn_sched_barrier(0);
        compute_block(ring[d]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Add the waves' partial sums through LDS, kRound fragments at a time;
  // wave w finishes fragments w, w + kW, ... of the round.  The first
  // barrier of a round also orders the previous round's (or unit's) reads
  // before the writes.
  template <typename Emit>
  __device__ __forceinline__ void reduce(const f32x4 (&acc)[kT], Emit&& emit) {
#pragma unroll
    for (int f0 = 0; f0 < kT; f0 += kRound) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kRound; ++q)
        if (f0 + q < kT) red[wave][q][lane] = acc[f0 + q];
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kRound; ++q) {
        if (f0 + q >= kT || q % kW != wave) continue;
        f32x4 v = red[0][q][lane];
#pragma unroll
        for (int w = 1; w < kW; ++w) v += red[w][q][lane];
        emit(f0 + q, v);
      }
    }
  }
};

template <int XD, int WD, int OD, int K16, int NS>
__global__ __launch_bounds__(kThreads) void shrink_split_h(const ShrinkParams p) {
  using Core = SplitHCore<XD, WD, K16, NS>;
  prefetch_params(p);
  extern __shared__ __align__(16) int32_t lds[];  // segment table, 4 * batches + 1 words
  __shared__ int32_t wave_total[kWaves];
  __shared__ typename Core::RedLds red;
  __shared__ typename Core::StageLds stage;
  const SegTable tab = seg_table(lds, p.batches);
  const int32_t U = build_tile_table(p, tab, wave_total, kTileRows);
  if (U == 0) return;
  uint32_t u, u_end;
  unit_range(p, (uint32_t)U, &u, &u_end);
  if (u >= u_end) return;

  Core core(p, red, stage);
  int b = last_at_most(tab.tile_start, p.batches + 1, (int32_t)u);
  for (; u < u_end; ++u) {
    while (uniform(tab.tile_start[b + 1]) <= (int32_t)u) ++b;
    const ShrinkUnit<NS> su = shrink_unit<NS>(p, tab, b, u, kTileRows);
    f32x4 acc[Core::kT];
    core.run(su, acc, p.steps);
    core.reduce(acc, [&](int i, f32x4 v) __attribute__((always_inline)) {
      shrink_store<OD, K16>(p, i, su.row0, su.rows, 0, core.j, core.g, v);
    });
  }
}

// ---------------------------------------------------------------------------
// Split-T: 64 tokens per unit, every wave runs all hidden steps, the lora_A
// blocks shared through LDS (the wave-to-tile assignment is at the kernel).
// ---------------------------------------------------------------------------

template <int XD, int K16, int NS>
struct SplitTBlock {
  using Sh = ShrinkShape<XD, K16, NS>;
  u32x4 x[Sh::kBlockT][Sh::kNV];     // this wave's input rows
  u32x4 a[NS][Sh::kPairs];           // this wave's share of the block's lora_A tiles
};

// The split-T contraction of one 64-token unit, shared by the shrink kernel
// and the fused shrink-expand kernel: `run` leaves in acc[h][i] this wave's
// fp32 sums (unscaled) of token tile tok_tile(h) and k tile k_tile(i) (k
// tile i of the launch is tile i % K16 of slice i / K16); lane (j, g) holds
// k = 16 (i % K16) + 4 g .. + 3 of token 16 tok_tile(h) + j.  The LDS
// staging buffers are the caller's (declared in the kernel).  P: a
// parameter block with the ShrinkParams fields x_row_bytes, H, steps and
// s[].a.
//
// With an even number of k tiles, at least 4, the waves form a 2 x 2 grid:
// wave w takes token tiles 2 (w % 2) and 2 (w % 2) + 1 and the k tiles of
// half w / 2.  Each lora_A fragment read from LDS then feeds two MFMAs and
// each input fragment kT / 2, so a step takes 2 + kT / 2 fragment reads
// per wave instead of 1 + kT.  Otherwise wave t takes token tile t and every
// k tile.  Either way each accumulator sees the same MFMAs in the same
// order.
template <int XD, int WD, int K16, int NS>
struct SplitTCore {
  using Sh = ShrinkShape<XD, K16, NS>;
  using Block = SplitTBlock<XD, K16, NS>;
  static constexpr int kT = Sh::kTiles;
  static constexpr int kB = Sh::kBlockT;
  static constexpr int kP = Sh::kPairs;
  static constexpr int xb = XD == F32 ? 4 : 2;
  static constexpr int kBuf = kT * kB;  // fragments of one block
  static constexpr bool kGrid = kT >= 4 && kT % 2 == 0;
  static constexpr int32_t kTurn = Sh::kRingT * kB;  // hidden steps per turn of the ring
  static constexpr int kTok = kGrid ? 2 : 1;       // token tiles per wave
  static constexpr int kKt = kGrid ? kT / 2 : kT;  // k tiles per wave
  static constexpr int kXBuf = kGrid ? 2 : 1;
  // lora_A fragments of a block per buffer: [buffer][tile i * kB + step][slot]
  // (see frag_slot); input fragments of a block by token tile (the tile
  // wave t loads); in the 2 x 2 grid two waves read each tile, so two
  // buffers as for lora_A, otherwise a tile is private to its wave and one
  // buffer does.
  typedef u32x4 ALds[2][kBuf][kFragSlots];
  typedef u32x4 XLds[kXBuf][kWaves][kB][kFragSlots];

  ALds& a_lds;
  XLds& x_lds;
  int lane, wave, tw, th, kh, g, j, lr, lb;
  int32_t H, h_steps;
  uint32_t xrb;
  uint32_t x_lane[2];
  int x_slot[2];
  uint32_t a_lane[kP];  // row offset + byte offset within the span
  int a_step[kP];       // step of this lane's 16 bytes within the block
  int a_frag[kP];       // fragment within a slice's part of the block, and slot
  int a_slot[kP];
  int r_slot;

  __device__ __forceinline__ int tok_tile(int h) const { return kGrid ? 2 * th + h : tw; }
  __device__ __forceinline__ int k_tile(int i) const { return (kGrid ? kh * kKt : 0) + i; }

  template <typename P>
  __device__ __forceinline__ SplitTCore(const P& p, ALds& a, XLds& x) : a_lds(a), x_lds(x) {
    lane = threadIdx.x & 63;
    wave = uniform(threadIdx.x >> 6);
    tw = wave;  // token tile this wave loads
    th = wave & 1;
    kh = wave >> 1;  // 2 x 2 grid: token pair, k half
    g = lane >> 4;
    j = lane & 15;
    H = p.H;
    h_steps = (H + 31) >> 5;  // hidden steps
    xrb = (uint32_t)p.x_row_bytes;  // 64 rows span < 2 GiB (host)
    // Input loads of a block, xq < kB: rows 16 tw + 8 (xq & 1) .. + 7 over
    // steps 2 (xq >> 1), + 1; lane l reads row + l / 8, elements 8 (l % 8) ..
    // of the span (hidden block l % 4 of step 2 (xq >> 1) + (l % 8) / 4).
    lr = lane >> 3;
    lb = lane & 7;
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2)
      x_lane[h2] = (uint32_t)(16 * tw + 8 * h2 + lr) * xrb + (uint32_t)(8 * lb * xb);
    x_slot[0] = frag_slot(lr, lb & 3);
    x_slot[1] = frag_slot(8 + lr, lb & 3);
    // This wave's lora_A loads of every slice's block: load pr = 4 q + tw
    // covers rows 16 kt + 8 half .. + 7 over steps 2 sp, 2 sp + 1 of the
    // block (kt = pr / kB, half and sp from pr % kB); lane l reads row +
    // l / 8, bytes 16 (l % 8) of the 128-byte span, which is hidden block
    // l % 4 of step 2 sp + (l % 8) / 4.
#pragma unroll
    for (int q = 0; q < kP; ++q) {
      const int pr = kWaves * q + tw;
      const int kt = pr / kB, r = pr % kB;
      const int half = r & 1, sp = r >> 1;
      const int row = 16 * kt + 8 * half + lr;
      a_lane[q] = (uint32_t)row * (uint32_t)H * 2u + (uint32_t)(16 * lb);
      a_step[q] = 2 * sp + (lb >> 2);
      a_frag[q] = kt * kB + a_step[q];
      a_slot[q] = frag_slot(8 * half + lr, lb & 3);
    }
    r_slot = frag_slot(j, g);  // this lane's slot when reading a fragment
  }

  // Hidden steps [s_lo, s_hi) of the unit (s_lo a multiple of kB; the
  // whole unit is [0, steps)); loads at or past min(s_hi, hidden steps)
  // read nothing, so their MFMAs add zeros.
  __device__ __forceinline__ void run(const ShrinkUnit<NS>& su, f32x4 (&acc)[kTok][kKt],
                                      int32_t s_lo, int32_t s_hi) {
    const int32_t lim = s_hi < h_steps ? s_hi : h_steps;
    auto load_block = [&](Block& blk, int32_t v0) __attribute__((always_inline)) {
#pragma unroll
      for (int xq = 0; xq < kB; ++xq) {
        // the lane's 8 elements: step 2 (xq >> 1) + lb / 4 of the block
        const int32_t step = v0 + 2 * (xq >> 1) + (lb >> 2);
        const bool ok = step < lim && 32 * step + 8 * (lb & 3) < H;
        const uint32_t span = (uint32_t)(32 * (step - (lb >> 2)) * xb);
        buf_load8<XD, kStreamLoad>(su.x, ok ? x_lane[xq & 1] + span : kOut, blk.x[xq]);
      }
#pragma unroll
      for (int q = 0; q < kP; ++q) {
        // the 128-byte span starts at the block's step 2 sp (even)
        const int32_t step = v0 + a_step[q];
        const bool ok = step < lim && 32 * step + 8 * (lb & 3) < H;
#pragma unroll
        for (int s = 0; s < NS; ++s)
          buf_load8<WD>(su.a[s], ok ? a_lane[q] + (uint32_t)(64 * (step - (lb >> 2))) : kOut,
                        &blk.a[s][q]);
      }
    };
    auto publish = [&](const Block& blk, int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int q = 0; q < kP; ++q)
          a_lds[buf][s * K16 * kB + a_frag[q]][a_slot[q]] = blk.a[s][q];
      // float32 inputs are rounded to the weight dtype here
#pragma unroll
      for (int xq = 0; xq < kB; ++xq)
        x_lds[kGrid ? buf : 0][wave][2 * (xq >> 1) + (lb >> 2)][x_slot[xq & 1]] =
            x_operand<XD, WD>(blk.x[xq]);
      __syncthreads();
    };
#pragma unroll
    for (int h = 0; h < kTok; ++h)
#pragma unroll
      for (int i = 0; i < kKt; ++i) acc[h][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute_block = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
      for (int st = 0; st < kB; ++st) {
        u32x4 xo[kTok];
#pragma unroll
        for (int h = 0; h < kTok; ++h)
          xo[h] = x_lds[kGrid ? buf : 0][kGrid ? 2 * th + h : wave][st][r_slot];
#pragma unroll
        for (int i = 0; i < kKt; ++i) {
          const u32x4 af = a_lds[buf][((kGrid ? kh * kKt : 0) + i) * kB + st][r_slot];
#pragma unroll
          for (int h = 0; h < kTok; ++h) acc[h][i] = mfma<WD>(af, xo[h], acc[h][i]);
        }
      }
    };

    // A ring of kD blocks in registers: block n + kD - 1 is issued, then
    // block n is published to LDS buffer n % 2 (kD is even) and computed.
    // The barrier in publish also orders every wave's reads of a buffer
    // (block n - 2) before it is written again.  Loads past the hidden
    // steps read nothing.
    constexpr int kD = Sh::kRingT;
    static_assert(kD % 2 == 0, "LDS buffers alternate with the ring");
    Block ring[kD];
#pragma unroll
    for (int d = 0; d + 1 < kD; ++d) {
      load_block(ring[d], s_lo + d * kB);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int32_t s = s_lo; s < s_hi; s += kD * kB) {
#pragma unroll
      for (int d = 0; d < kD; ++d) {
        load_block(ring[(d + kD - 1) % kD], s + (d + kD - 1) * kB);
        __builtin_amdgcn_sched_barrier(0);
        publish(ring[d], d & 1);
        compute_block(d & 1);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

// Cache policy of the parts workspace accesses: device scope (sc1), as
// atomics at that scope use, so that every XCD sees them in memory.
constexpr int kDevScope = 0x10;

// Balanced split-T (limits::part_plan): this workgroup's part `part` of P of
// an overflow unit has its fp32 sums in acc.  Publish them to part slot q
// (q - part .. q - part + P - 1 are the unit's parts) of the workspace, wait
// until they are written, and count the part in at the unit's counter.
// The last part to arrive clears the counter, puts in sum the sum of all P
// parts' slots taken in part order (the same order and values whichever
// part ends last) and returns true; the others return false and leave.
// Slot layout: [wave][token tile h][k tile i][lane], 16 bytes each.
template <typename Core>
__device__ __forceinline__ bool reduce_parts(const ShrinkParams& p, uint32_t P, uint32_t e,
                                             uint32_t part, uint32_t q, int32_t* flag,
                                             const f32x4 (&acc)[Core::kTok][Core::kKt],
                                             f32x4 (&sum)[Core::kTok][Core::kKt]) {
  constexpr int kTok = Core::kTok, kKt = Core::kKt;
  static_assert(kWaves * kTok * kKt * 1024 <= (int)limits::kShrinkPartBytes, "part slot size");
  uint32_t* counters = static_cast<uint32_t*>(p.ws);
  char* slots = static_cast<char*>(p.ws) + limits::shrink_workspace_counter_bytes(p.cus);
  const int lane = threadIdx.x & 63, wave = uniform(threadIdx.x >> 6);
  auto slot_off = [&](int h, int i) __attribute__((always_inline)) {
    return (uint32_t)(((wave * kTok + h) * kKt + i) * 1024 + lane * 16);
  };
  {
    const rsrc_t mine = make_rsrc(slots + (int64_t)q * limits::kShrinkPartBytes,
                                  limits::kShrinkPartBytes);
#pragma unroll
    for (int h = 0; h < kTok; ++h)
#pragma unroll
      for (int i = 0; i < kKt; ++i)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[h][i]), mine,
                                               (int)slot_off(h, i), 0, kDevScope);
  }
  // every wave's slot stores complete before the count
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = (int32_t)__hip_atomic_fetch_add(&counters[e], 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (uniform(*flag) != (int32_t)P - 1) return false;
  if (threadIdx.x == 0)
    __hip_atomic_store(&counters[e], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // Sum in part order, reading every part (this one's too, written above)
  // back from the workspace, so that acc (the MFMA accumulators) is dead;
  // kR parts' loads in flight.
  constexpr int kR = kTok * kKt <= 8 ? 2 : 1;
  const uint32_t first = q - part;
  for (uint32_t r0 = 0; r0 < P; r0 += kR) {
    f32x4 v[kR][kTok][kKt];
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      const uint32_t r = r0 + k < P ? r0 + k : r0;
      const rsrc_t slot = make_rsrc(slots + (int64_t)(first + r) * limits::kShrinkPartBytes,
                                    limits::kShrinkPartBytes);
#pragma unroll
      for (int h = 0; h < kTok; ++h)
#pragma unroll
        for (int i = 0; i < kKt; ++i)
          v[k][h][i] = __builtin_bit_cast(
              f32x4,
              __builtin_amdgcn_raw_buffer_load_b128(slot, (int)slot_off(h, i), 0, kDevScope));
    }
#pragma unroll
    for (int k = 0; k < kR; ++k) {
      if (r0 + k < P) {
#pragma unroll
        for (int h = 0; h < kTok; ++h)
#pragma unroll
          for (int i = 0; i < kKt; ++i)
            sum[h][i] = r0 + k == 0 ? v[k][h][i] : sum[h][i] + v[k][h][i];
      }
    }
  }
  return true;
}

template <int XD, int WD, int OD, int K16, int NS>
__global__ __launch_bounds__(kThreads) void shrink_split_t(const ShrinkParams p) {
  using Core = SplitTCore<XD, WD, K16, NS>;
  prefetch_params(p);
  extern __shared__ __align__(16) int32_t lds[];  // segment table, 4 * batches + 1 words
  __shared__ int32_t wave_total[kWaves];
  __shared__ typename Core::ALds a_lds;
  __shared__ typename Core::XLds x_lds;
  const SegTable tab = seg_table(lds, p.batches);
  const int32_t U = build_tile_table(p, tab, wave_total, kShrinkTokensSplitT);
  if (U == 0) return;
  // Units, and the hidden steps of each, this workgroup runs: unit_span, or
  // (a workspace; limits::part_plan) one whole unit on each of the first W
  // workgroups and the parts of the other units on the next ones.
  const uint32_t C = (uint32_t)p.cus;
  const limits::PartPlan plan =
      p.ws ? limits::part_plan((uint32_t)U, C, (uint32_t)p.grid, (uint32_t)((p.H + 31) >> 5))
           : limits::PartPlan{0, 0, 0};
  const uint32_t W = plan.W;
  uint32_t u, u_end, q = 0, part = 0;
  int32_t s_lo = 0, s_hi = p.steps;
  if (plan.P == 0) {
    unit_range(p, (uint32_t)U, &u, &u_end);
  } else if (blockIdx.x < W) {
    const limits::UnitSpan sp = limits::unit_span(W, W, C, blockIdx.x);
    u = sp.begin;
    u_end = sp.end;
  } else {
    const limits::PartItem it = limits::part_item(plan, blockIdx.x);
    if (!it.valid) return;
    u = it.unit;
    u_end = u + 1;
    part = it.part;
    q = (u - W) * plan.P + part;
    const limits::StepSpan ss = limits::part_steps(part, plan.P, (uint32_t)((p.H + 31) >> 5));
    s_lo = ss.lo;
    s_hi = ss.hi;
  }
  if (u >= u_end) return;

  Core core(p, a_lds, x_lds);
  int b = last_at_most(tab.tile_start, p.batches + 1, (int32_t)u);
  auto store_unit = [&](int32_t row0, int32_t rows, const f32x4 (&v)[Core::kTok][Core::kKt])
      __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < Core::kTok; ++h)
#pragma unroll
      for (int i = 0; i < Core::kKt; ++i)
        shrink_store<OD, K16>(p, core.k_tile(i), row0, rows, 16 * core.tok_tile(h), core.j,
                              core.g, v[h][i]);
  };
  // A part (one unit, hidden steps [s_lo, s_hi)) leaves the loop after its
  // contraction and reduces outside it, where no register the loop keeps
  // live is needed.
  const bool is_part = plan.P != 0 && blockIdx.x >= W;
  f32x4 acc[Core::kTok][Core::kKt];
  int32_t row0 = 0, rows = 0;
  for (; u < u_end; ++u) {
    while (uniform(tab.tile_start[b + 1]) <= (int32_t)u) ++b;
    const ShrinkUnit<NS> su = shrink_unit<NS>(p, tab, b, u, kShrinkTokensSplitT);
    core.run(su, acc, s_lo, s_hi);
    if (is_part) {
      row0 = su.row0;
      rows = su.rows;
      break;
    }
    store_unit(su.row0, su.rows, acc);
  }
  if (is_part) {
    f32x4 sum[Core::kTok][Core::kKt];
    if (reduce_parts<Core>(p, plan.P, u - W, part, q, &wave_total[0], acc, sum))
      store_unit(row0, rows, sum);
  }
}

// Any shape, stride and alignment: one output element per thread and
// iteration, fp32 fused multiply-adds over the hidden dimension.
template <int XD, int WD, int OD>
__global__ __launch_bounds__(kThreads) void shrink_generic(const ShrinkParams p) {
  prefetch_params(p);
  extern __shared__ __align__(16) int32_t lds[];
  __shared__ int32_t wave_total[kWaves];
  const SegTable tab = seg_table(lds, p.batches);
  const int32_t U = build_tile_table(p, tab, wave_total, kTileRows);
  const int32_t K = p.K;
  const int64_t per_unit = (int64_t)kTileRows * K * p.num_slices;
  for (int32_t u = blockIdx.x; u < U; u += p.grid) {
    const int b = last_at_most(tab.tile_start, p.batches + 1, u);
    const int64_t row0 = uniform(tab.seg_row[b]) + (int64_t)(u - uniform(tab.tile_start[b])) *
                                                       kTileRows;
    const int64_t rows = uniform(tab.seg_end[b]) - row0;
    const int64_t a = uniform(tab.seg_lora[b]);
    for (int64_t e = threadIdx.x; e < per_unit; e += kThreads) {
      const int si = (int)(e / ((int64_t)kTileRows * K));
      const int64_t rem = e - (int64_t)si * kTileRows * K;
      const int64_t r = rem / K, k = rem - r * K;
      if (r >= rows) continue;
      const int64_t t = row0 + r;
      const char* xrow = static_cast<const char*>(p.x) + t * p.x_row_bytes;
      const uint16_t* arow = static_cast<const uint16_t*>(p.s[si].a) + (a * K + k) * p.H;
      float acc = 0.f;
      for (int32_t h = 0; h < p.H; ++h) {
        float xv;
        if constexpr (XD == F32) {
          const float f = reinterpret_cast<const float*>(xrow)[h];
          xv = widen<WD>(pack2<WD>(f, 0.f) & 0xFFFFu);  // rounded to the weight dtype
        } else {
          xv = widen<XD>(reinterpret_cast<const uint16_t*>(xrow)[h]);
        }
        acc = __builtin_fmaf(xv, widen<WD>(arow[h]), acc);
      }
      const float v = acc * p.scale;
      char* orow = static_cast<char*>(p.s[si].out) + t * p.s[si].out_row_bytes;
      if constexpr (OD == F32)
        reinterpret_cast<float*>(orow)[k] = v;
      else
        reinterpret_cast<uint16_t*>(orow)[k] = (uint16_t)(pack2<OD>(v, 0.f) & 0xFFFFu);
    }
  }
}

// ---------------------------------------------------------------------------
// Kernel tables.
// ---------------------------------------------------------------------------

template <int XD, int WD, int OD, int K16, int NS>
const void* shrink_entry(bool split_t) {
  if constexpr (K16 * NS > 16) {
    return nullptr;
  } else {
    return split_t ? reinterpret_cast<const void*>(&shrink_split_t<XD, WD, OD, K16, NS>)
                   : reinterpret_cast<const void*>(&shrink_split_h<XD, WD, OD, K16, NS>);
  }
}

template <int XD, int WD, int OD, int K16>
const void* shrink_by_ns(int ns, bool split_t) {
  switch (ns) {
    case 1: return shrink_entry<XD, WD, OD, K16, 1>(split_t);
    case 2: return shrink_entry<XD, WD, OD, K16, 2>(split_t);
    case 3: return shrink_entry<XD, WD, OD, K16, 3>(split_t);
    default: return nullptr;
  }
}

template <int XD, int WD, int K16>
const void* shrink_by_out(int od, int ns, bool split_t) {
  switch (od) {
    case F16: return shrink_by_ns<XD, WD, F16, K16>(ns, split_t);
    case BF16: return shrink_by_ns<XD, WD, BF16, K16>(ns, split_t);
    case F32: return shrink_by_ns<XD, WD, F32, K16>(ns, split_t);
    default: return nullptr;
  }
}

template <int K16>
const void* shrink_table(int xd, int wd, int od, int ns, bool split_t) {
  if (wd == BF16 && xd == BF16) return shrink_by_out<BF16, BF16, K16>(od, ns, split_t);
  if (wd == BF16 && xd == F32) return shrink_by_out<F32, BF16, K16>(od, ns, split_t);
  if (wd == F16 && xd == F16) return shrink_by_out<F16, F16, K16>(od, ns, split_t);
  if (wd == F16 && xd == F32) return shrink_by_out<F32, F16, K16>(od, ns, split_t);
  return nullptr;
}

}  // namespace dev
}  // namespace sgmv

// sgmv_device.h -- gfx950 device code for SGMV expand-slice (included by the
// kernel translation units; internal to libsgmv).
//
// Operation (wiki page "Implementation: Predibase Lorax SGMV Expand Slice
// Kernel", Description and I/O Contract): for segment b with adapter
// a = idx[b] != -1 and each row t of the segment,
//     out[t][off + n] (+)= sum_k x[t][k] * W[a][n][k],   n in [0, N).
//
// Design (MI355X-first; the page's Triton GroupGEMM tiling is prior art only):
//
//  * One persistent launch.  Every workgroup first scans the segment
//    metadata (device int64 arrays, never read back by the host) into an LDS
//    table of row-tile prefix sums, row ranges and adapters -- the
//    device-side scheduler.  Index -1 segments and segments outside [0, T)
//    get no tiles.
//  * Work unit = (column tile of 256 output columns, 16-row tile of one
//    segment).  The column tiles are split into 8 groups, one per XCD
//    (workgroup ids are dealt round-robin to the XCDs); a group's units are
//    walked band of row tiles by band, column tile by column tile, so
//    consecutive units of a workgroup run down the rows of a segment under
//    one column tile and the adapter's weight tile stays in registers.  The
//    workgroups of an XCD take interleaved chunks of that walk and so share
//    input rows and weight tiles through the XCD's L2.
//  * Each of the 4 wavefronts owns 64 of the 256 columns.  The contraction
//    runs on the matrix cores as C^T = W . X^T with v_mfma_f32_16x16x32_
//    {bf16,f16}: the weight rows are the MFMA rows (A operand, stationary in
//    VGPRs), the 16 tokens of the tile are the MFMA columns (B operand).
//    Weight rows are assigned to MFMA rows so that every lane ends up holding
//    8 consecutive output columns of one token.
//  * Rank step ks of the MFMA covers rank [32 ks, 32 ks + 32); lane group g
//    loads the 16-byte block 32 ks + 8 g of its token's input row and of its
//    weight row.
//  * The prior output is read and the result written row-wise (a row's 128
//    bytes, 256 for float32, per instruction) and moved to and from the
//    accumulator layout through a small per-wave LDS tile.  The stores are
//    non-temporal at device scope: every output line is written once and not
//    read again by the call.
//  * fp32 accumulation; with add_inputs the prior output seeds the
//    accumulator, so the result is rounded once (v_cvt_pk_{bf16,f16}_f32,
//    nearest even).  float32 inputs are rounded to the weight dtype first.
//
// Two kernels share this structure:
//  * expand_fast: software-pipelined.  The next unit's loads are issued
//    before the current unit's contraction and stores.  Every unit issues
//    the same vector-memory instructions (addresses of lanes that have no
//    data are clamped to valid locations, their values are masked in
//    registers and their stores are predicated), so the compiler can wait
//    for one unit's data with a nonzero vmcnt instead of draining the queue
//    -- on gfx9 the counter covers loads and stores alike and retires in
//    issue order.  Needs rank % 8 == 0, slice widths % 8 == 0 and 16-byte
//    alignment of rows and column groups.
//  * expand_generic: any shape, stride and alignment (element-wise edges),
//    any rank (rank processed in 32-wide chunks, weights reloaded per unit).
#pragma once

#include "sgmv_common.h"
#include "sgmv_launch.h"

// Largest rank-step count (rank <= 32 * steps) whose fast kernels keep a
// second weight tile in registers to prefetch across adapter / column-tile
// changes.
#ifndef SGMV_DOUBLE_W_MAX_KSTEPS
#define SGMV_DOUBLE_W_MAX_KSTEPS 2
#endif

namespace sgmv {
namespace dev {

// Unit counts, unit indices and row-tile counts are below 2^31 (the host
// refuses larger problems), so the scheduler's arithmetic is 32-bit: 64-bit
// division is a long scalar sequence that every wave of a compute unit would
// queue for on the shared scalar ALU.
//
// First column tile of column group g (g = kColumnGroups: one past the last).
__device__ __forceinline__ int column_group_tile(const Params& p, int g) {
  return (int)((uint32_t)p.total_tiles * (uint32_t)g / kColumnGroups);
}

__device__ __forceinline__ int slice_of(const Params& p, int tile) {
  int si = 0;
  while (si + 1 < p.num_slices && p.s[si + 1].tile_begin <= tile) ++si;
  return si;
}

// One work unit as one wavefront sees it.
struct Unit {
  int64_t col0;    // first of the wave's 64 columns, within the slice
  int64_t a;       // adapter
  int64_t t;       // this lane's output row (token j of the tile)
  int64_t seg_t0;  // first row of the segment (a valid row for clamping)
  int tile;        // global column tile
  int si;          // slice
  bool row_ok;     // token j lies inside the segment
};

// Wave-uniform walk over the units of a range, column-tile-major; the
// segment's row range and adapter come from the LDS table.
struct Cursor {
  const Params& p;
  const SegTable& tab;
  int32_t RT, rt;
  int tile, b, si;

  __device__ __forceinline__ Cursor(const Params& p_, const SegTable& t, int32_t rt_total,
                                    uint32_t u)
      : p(p_), tab(t), RT(rt_total) {
    tile = (int)(u / (uint32_t)RT);
    rt = (int32_t)(u - (uint32_t)tile * (uint32_t)RT);
    b = last_at_most(tab.tile_start, p.batches + 1, rt);
    while (uniform(tab.tile_start[b + 1]) <= rt) ++b;
    si = slice_of(p, tile);
  }

  __device__ __forceinline__ void advance() {
    if (++rt == RT) {
      rt = 0;
      ++tile;
      b = 0;
      si = slice_of(p, tile);
    }
    while (uniform(tab.tile_start[b + 1]) <= rt) ++b;
  }

  __device__ __forceinline__ Unit decode(int wave, int j) const {
    const int64_t seg_row = uniform(tab.seg_row[b]);
    const int64_t seg_end = uniform(tab.seg_end[b]);
    const SliceDesc& S = p.s[si];
    Unit u;
    u.tile = tile;
    u.si = si;
    u.col0 = (int64_t)(tile - S.tile_begin) * kTileCols + wave * kWaveCols;
    u.a = uniform(tab.seg_lora[b]);
    u.t = seg_row + (int64_t)(rt - uniform(tab.tile_start[b])) * kTileRows + j;
    u.row_ok = u.t < seg_end;
    u.seg_t0 = seg_row;
    return u;
  }
};

// Weight row held by MFMA row i = j of subtile s = 2q + h: the accumulator
// rows of lane group g are then the 8 consecutive output columns
// col0 + 32q + 8g + 0..7.
__device__ __forceinline__ int64_t weight_row(int64_t col0, int s, int j) {
  return col0 + 32 * (s >> 1) + 8 * (j >> 2) + 4 * (s & 1) + (j & 3);
}

// ---------------------------------------------------------------------------
// Fast kernel.
// ---------------------------------------------------------------------------

// One unit of the fast kernel: scalar (wave-uniform) resources over the
// unit's valid input rows and the wave's output block, and the weight tile
// it needs.
// Adapter indices, columns within a slice and segment row counts fit in 32
// bits on the fast path (its output rows span less than 2 GiB per 16 rows),
// which keeps the scalar state of the pipelined loop small.
struct FastUnit {
  rsrc_t x;       // inputs: the tile's valid rows (rows past the segment read zero)
  rsrc_t o;       // output: from (row0, off + col0) to the end of the last valid row's block
  uint32_t lx;     // gathered tiles: this lane's input row offset (kOut: none)
  uint32_t lro[4]; // gathered tiles: this lane's output offset per row-wise access (kOut: none)
  int32_t a;      // adapter
  int32_t col0;   // first of the wave's 64 columns, within the slice
  int32_t n_rem;  // slice columns left from col0 (<= 0: the wave has none)
  int tile;       // global column tile
  int si;         // slice
};

// Walk of the fast kernels over their unit range.  Order: column group
// (kColumnGroups contiguous ranges of column tiles, one per XCD), then band
// of band_tiles row tiles, then column tile, then row tile.  Within a run of
// row tiles of one segment under one column tile, a step only advances row
// offsets; segment, tile and band changes re-read the LDS table.
template <bool GATHER>
struct Walk {
  const Params& p;
  const SegTable& tab;      // segment tiles (not GATHER)
  const GatherTable& gt;    // gathered tiles (GATHER)
  int32_t* rows;            // GATHER: this wave's 16 token rows of the current tile
  int32_t RT;       // row tiles
  int wave;
  int ob;           // bytes per output element
  // position
  int gi, tile_lo, tile_hi;   // column group and its tiles [lo, hi)
  int32_t band_lo, band_hi;   // band's row tiles [lo, hi)
  int band_b;                 // segment holding band_lo
  int tile, si, b;           // b: table slot, or (GATHER) the tile's adapter
  int32_t rt;
  int32_t seg_tile_end;       // first row tile after segment b
  // run state for (tile, b) at row tile rt
  const char* x_row;          // inputs: first row of the row tile
  const char* o_row;          // output: first row, first column of the wave's block
  int32_t rows_left;          // segment rows from the tile's first row on
  int32_t a, col0;
  // this workgroup's chunks (see the fast kernel): units left in the current
  // chunk after the current unit, and the next chunk's offset in the group
  uint32_t c_left, next_off, g_base, g_size, chunk, stride;
  int32_t n_rem;

  __device__ __forceinline__ int group_tile(int g) const { return column_group_tile(p, g); }

  // Table slot holding row tile r, searching forward from slot `from` (a slot
  // at or before it).  Slots without tiles come before the slot that holds
  // the tile, so the last slot whose prefix is <= r is the one.
  __device__ __forceinline__ int slot_of(int32_t r, int from) const {
    int s = from;
    while (uniform(tab.tile_start[s + 1]) <= r) ++s;
    return s;
  }

  // GATHER: the adapter whose tiles hold row tile r (adapters without tokens
  // share the prefix of the next one, so the last prefix <= r is the owner).
  __device__ __forceinline__ int adapter_of(int32_t r) const {
    return last_at_most(gt.a_tiles, p.L + 1, r);
  }

  // GATHER: rows of tokens 16 k .. 16 k + 15 of adapter a, in token order,
  // into rows[0 ..): one ballot per 64 tokens of the table.
  __device__ __forceinline__ void fetch_rows(int a, int32_t k) const {
    const int lane = threadIdx.x & 63;
    const int32_t lo = kTileRows * k, hi = lo + kTileRows;
    int32_t seen = 0;
    for (int c = 0; c < p.batches && seen < hi; c += 64) {
      const int t = c + lane;
      const bool m = t < p.batches && gt.tok_a[t] == a;
      const uint64_t mask = __ballot(m);
      const int32_t r = seen + (int32_t)__builtin_amdgcn_mbcnt_hi(
                                   (uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
      if (m && r >= lo && r < hi) rows[r - lo] = t;
      seen += (int32_t)__builtin_popcountll(mask);
    }
  }

  __device__ __forceinline__ Walk(const Params& p_, const SegTable& t, const GatherTable& g,
                                  int32_t* rows_, int32_t rt_total, int wave_, int ob_,
                                  uint32_t u)
      : p(p_), tab(t), gt(g), rows(rows_), RT(rt_total), wave(wave_), ob(ob_) {
    seek(u);
  }

  // Move to the next unit of the workgroup: the rest of the current chunk,
  // else the start of the next chunk.  False when there is none.
  __device__ __forceinline__ bool next() {
    if (c_left > 0) {
      advance();
      --c_left;
      return true;
    }
    if (next_off < g_size) {
      seek(g_base + next_off);
      c_left = (g_size - next_off < chunk ? g_size - next_off : chunk) - 1;
      next_off += stride;
      return true;
    }
    return false;
  }

  // Position on unit u (any unit of the launch).
  __device__ __forceinline__ void seek(uint32_t u) {
    // group: units of group g start at group_tile(g) * RT
    const uint32_t rt_n = (uint32_t)RT;
    gi = 0;
    while (gi + 1 < kColumnGroups && (uint32_t)group_tile(gi + 1) * rt_n <= u) ++gi;
    tile_lo = group_tile(gi);
    tile_hi = group_tile(gi + 1);
    const uint32_t nt = (uint32_t)(tile_hi - tile_lo);
    const uint32_t v = u - (uint32_t)tile_lo * rt_n;
    const uint32_t RB = (uint32_t)p.band_tiles;
    const uint32_t nb = (rt_n + RB - 1) / RB;
    uint32_t bi = v / (RB * nt);
    if (bi > nb - 1) bi = nb - 1;
    band_lo = (int32_t)(bi * RB);
    band_hi = band_lo + p.band_tiles < RT ? band_lo + p.band_tiles : RT;
    const uint32_t w = v - (uint32_t)band_lo * nt;
    const uint32_t rb = (uint32_t)(band_hi - band_lo);
    const uint32_t wq = w / rb;
    tile = tile_lo + (int)wq;
    rt = band_lo + (int32_t)(w - wq * rb);
    if constexpr (GATHER) {
      b = adapter_of(rt);
    } else {
      band_b = last_at_most(tab.tile_start, p.batches + 1, band_lo);
      b = slot_of(rt, band_b);
    }
    si = slice_of(p, tile);
    new_run();
  }

  __device__ __forceinline__ void new_run() {
    const SliceDesc& S = p.s[si];
    col0 = (int64_t)(tile - S.tile_begin) * kTileCols + wave * kWaveCols;
    const int64_t n_left = S.n - col0;
    n_rem = n_left <= 0 ? 0 : (n_left > kWaveCols ? kWaveCols : (int32_t)n_left);
    if constexpr (GATHER) {
      // row tile rt is tile k of adapter b; each lane takes its token's row
      // from rows (see the fast kernel)
      const int32_t k = rt - uniform(gt.a_tiles[b]);
      const int32_t left = uniform(gt.a_count[b]) - kTileRows * k;
      rows_left = left < kTileRows ? left : kTileRows;
      a = b;
      seg_tile_end = rt + 1;
      x_row = static_cast<const char*>(S.x);
      o_row = static_cast<const char*>(p.out) + (S.offset + col0) * ob;
      fetch_rows(b, k);
      return;
    }
    const int64_t seg_row = uniform(tab.seg_row[b]);
    const int64_t seg_end = uniform(tab.seg_end[b]);
    a = uniform(tab.seg_lora[b]);
    seg_tile_end = uniform(tab.tile_start[b + 1]);
    const int64_t row0 = seg_row + (int64_t)(rt - uniform(tab.tile_start[b])) * kTileRows;
    rows_left = (int32_t)(seg_end - row0);
    x_row = static_cast<const char*>(S.x) + row0 * S.x_row_bytes;
    o_row = static_cast<const char*>(p.out) + row0 * p.out_row_bytes + (S.offset + col0) * ob;
  }

  __device__ __forceinline__ void advance() {
    ++rt;
    if (rt == band_hi) {
      ++tile;
      if (tile == tile_hi) {  // next band of the group (or next group)
        band_lo = band_hi;
        if (band_lo == RT) {
          do {
            ++gi;
            tile_lo = group_tile(gi);
            tile_hi = group_tile(gi + 1);
          } while (tile_lo == tile_hi && gi + 1 < kColumnGroups);
          band_lo = 0;
          b = 0;
        }
        band_hi = band_lo + p.band_tiles < RT ? band_lo + p.band_tiles : RT;
        tile = tile_lo;
        if constexpr (!GATHER) band_b = slot_of(band_lo, b);
      }
      rt = band_lo;
      b = GATHER ? adapter_of(rt) : band_b;
      si = slice_of(p, tile);
      new_run();
    } else if (rt == seg_tile_end) {
      if constexpr (GATHER) {
        while (uniform(gt.a_tiles[b + 1]) <= rt) ++b;  // the next tile's adapter
      } else {
        ++b;
        while (uniform(tab.tile_start[b + 1]) <= rt) ++b;
      }
      new_run();
    } else {
      x_row += kTileRows * p.s[si].x_row_bytes;
      o_row += kTileRows * p.out_row_bytes;
      rows_left -= kTileRows;
    }
  }
};

// Fast-kernel variants by KS: rank <= 32 KS for KS >= 1, with the input tile
// shared by the workgroup's waves through LDS; KS = 0 is rank <= 16 with one
// rank step and no sharing -- each wave loads its own (small) input tile,
// which beats a barrier per unit when workgroups have only a unit or two.
template <int KS>
struct FastShape {
  static constexpr int kSteps = KS == 0 ? 1 : KS;  // 32-wide rank steps
  static constexpr bool kShareX = KS != 0;
  static constexpr int kChunks = kShareX ? (kSteps + kWaves - 1) / kWaves : 1;
};

// Loads of one unit that are in flight while the previous unit computes:
// the rank chunks of the input tile this wave loads (shared: chunk ks = wave
// + 4 i, 16 rows x 32 rank in MFMA operand order, for the workgroup) and the
// prior output of the wave's own block.
template <int XD, int OD, int KS>
struct Stage {
  u32x4 x[FastShape<KS>::kChunks * raw_vecs<XD>()];
  u32x4 o[2 * raw_vecs<OD>()];    // prior output: two 8-column groups
};

// GATHER: per-token calls whose row tiles gather up to 16 tokens of one
// adapter (rows not contiguous): each lane's row offset comes from the table.
template <int XD, int WD, int OD, bool ADD, int KS, bool GATHER>
__global__ __launch_bounds__(kThreads) void expand_fast(const Params p) {
  constexpr int kSteps = FastShape<KS>::kSteps;
  constexpr bool kShareX = FastShape<KS>::kShareX;
  prefetch_params(p);
  // segment table, 4 * batches + 1 words, or (GATHER) the gathered table,
  // batches + 2 L + 1 words
  extern __shared__ __align__(16) int32_t lds[];
  __shared__ int32_t wave_total[kWaves];
  const SegTable tab = seg_table(lds, p.batches);
  const GatherTable gt = gather_table(lds, p.batches, p.L);
  int32_t RT;
  if constexpr (GATHER) RT = build_gather_table(p, gt, wave_total);
  else RT = build_tile_table(p, tab, wave_total);
  const uint32_t U = (uint32_t)RT * (uint32_t)p.total_tiles;
  if (U == 0) return;

  // Work assignment.  With a grid of 8 k workgroups (k >= 2), workgroup i
  // serves column group i % 8 (its XCD, under the round-robin dispatch of
  // workgroups to XCDs) and takes the chunks i / 8, i / 8 + k, i / 8 + 2 k,
  // ... of `chunk` consecutive units of that group's walk.  The k workgroups
  // of an XCD thus sweep the walk side by side, within a window of about
  // k chunks, so its L2 holds the input rows and weight tiles they share;
  // inside a chunk the weight tile stays in registers.  chunk =
  // min(chunk_units, ceil(group units / k)): a group smaller than k chunk
  // units is cut into rounded-up shares, so some workgroups stay idle while
  // the rest hold two units or more, whose loads then overlap the previous
  // unit's work (faster, measured, than one unit on every workgroup).
  // chunk_units divides the walk's band height, so chunks do not straddle a
  // column tile's run of a band.  Otherwise one contiguous range per
  // workgroup.
  const uint32_t G = (uint32_t)p.grid;
  uint32_t c_start, c_len;     // current chunk: [c_start, c_start + c_len)
  uint32_t g_base = 0, g_size = 0, chunk = 0, stride = 0, next_off = 0;
  if (G >= 16 && (G & 7) == 0) {
    const int grp = blockIdx.x & 7;
    const int t_lo = column_group_tile(p, grp), t_hi = column_group_tile(p, grp + 1);
    g_base = (uint32_t)t_lo * (uint32_t)RT;
    g_size = (uint32_t)(t_hi - t_lo) * (uint32_t)RT;
    const uint32_t k = G >> 3;
    const uint32_t per_wg = (g_size + k - 1) / k;
    chunk = per_wg < (uint32_t)p.chunk_units ? (per_wg > 0 ? per_wg : 1) : (uint32_t)p.chunk_units;
    stride = k * chunk;
    const uint32_t s0 = (blockIdx.x >> 3) * chunk;
    if (s0 >= g_size) return;
    c_start = g_base + s0;
    c_len = g_size - s0 < chunk ? g_size - s0 : chunk;
    next_off = s0 + stride;
  } else {
    uint32_t u_end;
    unit_range(p, U, &c_start, &u_end);
    if (c_start >= u_end) return;
    c_len = u_end - c_start;
  }

  constexpr int xb = XD == F32 ? 4 : 2;
  constexpr int ob = OD == F32 ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);  // resources built from it stay scalar
  const int g = lane >> 4;   // lane group: rank sub-block / column group
  const int j = lane & 15;   // token of the tile / MFMA row of the A operand
  const int K = p.K;
  const int64_t os_bytes = p.out_row_bytes;

  // Rank step ks covers rank [32 ks, 32 ks + 32); lane group g holds the
  // 8-element block 32 ks + 8 g (the same grouping as the generic kernel, so
  // both give bit-identical results).  Blocks past K read zero.
  // Loop-invariant lane offsets of the weights: row weight_row(0, s, j) of
  // the tile.
  // Output tile of the wave (16 rows x 64 columns) in HBM: accessed
  // row-wise, kLPR lanes per row (a row's 128 bytes, 256 for float32, in one
  // instruction, against 64 bytes with the accumulator layout), and moved
  // between that layout and the MFMA accumulator layout through a per-wave
  // LDS tile: 16-byte block b of row r in slot kNB r + (b ^ (r mod kNB)).
  // The LDS serves a 16-byte access 8 lanes at a time, free of bank
  // conflicts when they hit 8 slot classes mod 8: the 8 lanes of a row-wise
  // access share a row (blocks b ^ const), those of the accumulator layout
  // share a block over 8 consecutive rows (r mod 8 differs).  Access m
  // covers rows m kRPI .. + kRPI - 1; this lane reads or writes block oblk
  // of row m kRPI + orow -- at offset oc_off[m] for contiguous rows, or
  // (GATHER) at the unit's lro[m], from that row's token.
  constexpr int kNB = 64 * ob / 16;           // 16-byte blocks per tile row
  constexpr int kLPR = kNB;
  constexpr int kRPI = 64 / kLPR;
  constexpr int kOAcc = 2 * raw_vecs<OD>();   // row-wise accesses per tile
  static_assert(kOAcc * kRPI == kTileRows, "row-wise accesses cover the tile");
  __shared__ u32x4 o_lds[kWaves][kTileRows * kNB];
  auto o_slot = [](int r, int b) __attribute__((always_inline)) -> int {
    return kNB * r + (b ^ (r % kNB));
  };
  // accumulator-layout block of lane (j, g): column group q, vector v
  auto acc_blk = [&](int q, int v) __attribute__((always_inline)) -> int {
    return raw_vecs<OD>() == 1 ? 4 * q + g : 2 * (4 * q + g) + v;
  };
  const int orow = lane / kLPR, oblk = lane % kLPR;
  const int ocol = oblk * (16 / ob);          // first column of this lane's block
  static_assert(kOAcc <= 4, "FastUnit::lro holds the row-wise offsets");
  uint32_t oc_off[kOAcc];
#pragma unroll
  for (int m = 0; m < kOAcc; ++m)
    oc_off[m] = (uint32_t)((m * kRPI + orow) * os_bytes + oblk * 16);
  // offset of row-wise access m of unit u; blocks past the slice (only in a
  // slice's last column tile) take an out-of-range offset, as do rows past
  // the segment (outside the resource) or past a gathered tile's tokens
  auto o_at = [&](const FastUnit& u, int m) __attribute__((always_inline)) -> uint32_t {
    return ocol < u.n_rem ? (GATHER ? u.lro[m] : oc_off[m]) : kOut;
  };
  auto w_off = [&](int s, int ks) __attribute__((always_inline)) -> uint32_t {
    const int kb = 32 * ks + 8 * g;
    return kb < K ? (uint32_t)((weight_row(0, s, j) * K + kb) * 2) : kOut;
  };
  // Input tile: shared through LDS (KS >= 1): rank chunk ks (16 rows x 32
  // rank, one 16-byte block per lane in MFMA operand order) is loaded by wave
  // ks % 4 and read by all four.  Unshared (KS = 0): every wave loads chunk 0
  // itself.  Offsets depend on the slice's row stride.
  constexpr int kChunks = FastShape<KS>::kChunks;
  __shared__ u32x4 x_lds[2][kShareX ? kSteps : 1][64];
  uint32_t x_off[kChunks];
  int x_si = -1;
  auto x_chunk = [&](int i) __attribute__((always_inline)) -> int {
    return kShareX ? wave + kWaves * i : 0;
  };
  auto set_x_off = [&](int si) __attribute__((always_inline)) {
    const int64_t xs_bytes = p.s[si].x_row_bytes;
#pragma unroll
    for (int i = 0; i < kChunks; ++i) {
      const int kb = 32 * x_chunk(i) + 8 * g;
      x_off[i] = kb < K ? (uint32_t)((GATHER ? 0 : j * xs_bytes) + kb * xb) : kOut;
    }
    x_si = si;
  };

  __shared__ int32_t tile_rows[GATHER ? kWaves : 1][kTileRows];  // GATHER: token rows per wave
  Walk<GATHER> pos(p, tab, gt, tile_rows[GATHER ? wave : 0], RT, wave, ob, c_start);
  pos.c_left = c_len - 1;
  pos.next_off = next_off;
  pos.g_base = g_base;
  pos.g_size = g_size;
  pos.chunk = chunk;
  pos.stride = stride;
  auto next_unit = [&]() __attribute__((always_inline)) -> FastUnit {
    const int64_t rows = pos.rows_left < kTileRows ? pos.rows_left : kTileRows;
    FastUnit u;
    u.tile = pos.tile;
    u.si = pos.si;
    u.a = pos.a;
    u.col0 = pos.col0;
    u.n_rem = pos.n_rem;
    if constexpr (GATHER) {
      // Token j of the tile: this lane's row (the host keeps T rows of x and
      // of the output within 2 GiB, so row offsets fit 32 bits).
      const int64_t row = j < pos.rows_left ? pos.rows[j] : -1;
      u.lx = row >= 0 ? (uint32_t)(row * p.s[pos.si].x_row_bytes) : kOut;
      // row-wise output accesses: row m kRPI + orow of the tile, block oblk
#pragma unroll
      for (int m = 0; m < kOAcc; ++m) {
        const int r = m * kRPI + orow;
        u.lro[m] = r < pos.rows_left ? (uint32_t)(pos.rows[r] * p.out_row_bytes) + oblk * 16
                                     : kOut;
      }
      u.x = make_rsrc(pos.x_row, p.T * p.s[pos.si].x_row_bytes);
      u.o = make_rsrc(pos.o_row,
                      u.n_rem > 0 ? (p.T - 1) * p.out_row_bytes + (int64_t)u.n_rem * ob : 0);
    } else {
      u.lx = 0;
      u.x = make_rsrc(pos.x_row, rows * p.s[pos.si].x_row_bytes);
      u.o = make_rsrc(pos.o_row,
                      u.n_rem > 0 ? (rows - 1) * p.out_row_bytes + (int64_t)u.n_rem * ob : 0);
    }
    return u;
  };

  auto load_w = [&](u32x4 (&w)[4][kSteps], const FastUnit& u) __attribute__((always_inline)) {
    const SliceDesc& S = p.s[u.si];
    const rsrc_t r = make_rsrc(static_cast<const char*>(S.w) + (u.a * S.n + u.col0) * K * 2,
                               (int64_t)u.n_rem * K * 2);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int ks = 0; ks < kSteps; ++ks) buf_load8<WD>(r, w_off(s, ks), &w[s][ks]);
  };
  auto load_stage = [&](Stage<XD, OD, KS>& st, const FastUnit& u) __attribute__((always_inline)) {
    if (u.si != x_si) set_x_off(u.si);
#pragma unroll
    for (int i = 0; i < kChunks; ++i)
      if (x_chunk(i) < kSteps) buf_load8<XD>(u.x, u.lx + x_off[i], &st.x[i * raw_vecs<XD>()]);
    if constexpr (ADD) {
      // prior output, row-wise (st.o[m] = access m)
#pragma unroll
      for (int m = 0; m < kOAcc; ++m)
        st.o[m] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(u.o, o_at(u, m), 0, 0));
    }
  };
  // Publish this wave's chunks of a unit's input tile to LDS buffer `buf`
  // (float32 inputs are rounded to the weight dtype here) and wait for the
  // other waves' chunks.
  auto publish_x = [&](const Stage<XD, OD, KS>& st, int buf) __attribute__((always_inline)) {
    if constexpr (kShareX) {
#pragma unroll
      for (int i = 0; i < kChunks; ++i)
        if (x_chunk(i) < kSteps)
          x_lds[buf][x_chunk(i)][lane] = x_operand<XD, WD>(&st.x[i * raw_vecs<XD>()]);
      __syncthreads();
    }
  };
  auto compute_store = [&](const Stage<XD, OD, KS>& st, const u32x4 (&w)[4][kSteps],
                           const FastUnit& u, int buf) __attribute__((always_inline)) {
    f32x4 acc[4];
    if constexpr (ADD) {
      // row-wise prior output -> the wave's LDS tile -> accumulator layout
#pragma unroll
      for (int m = 0; m < kOAcc; ++m) o_lds[wave][o_slot(m * kRPI + orow, oblk)] = st.o[m];
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if constexpr (ADD) {
        u32x4 raw[raw_vecs<OD>()];
#pragma unroll
        for (int rv = 0; rv < raw_vecs<OD>(); ++rv) raw[rv] = o_lds[wave][o_slot(j, acc_blk(q, rv))];
        out_values<OD>(raw, v);
      }
      acc[2 * q] = f32x4{v[0], v[1], v[2], v[3]};
      acc[2 * q + 1] = f32x4{v[4], v[5], v[6], v[7]};
    }
#pragma unroll
    for (int ks = 0; ks < kSteps; ++ks) {
      u32x4 xo;
      if constexpr (kShareX) xo = x_lds[buf][ks][lane];
      else xo = x_operand<XD, WD>(&st.x[0]);
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[s] = mfma<WD>(w[s][ks], xo, acc[s]);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const float v[8] = {acc[2 * q][0], acc[2 * q][1], acc[2 * q][2], acc[2 * q][3],
                          acc[2 * q + 1][0], acc[2 * q + 1][1], acc[2 * q + 1][2],
                          acc[2 * q + 1][3]};
      u32x4 raw[raw_vecs<OD>()];
      out_pack<OD>(v, raw);
#pragma unroll
      for (int rv = 0; rv < raw_vecs<OD>(); ++rv) o_lds[wave][o_slot(j, acc_blk(q, rv))] = raw[rv];
    }
    // the wave's LDS tile -> row-wise stores (same column and row clamps)
#pragma unroll
    for (int m = 0; m < kOAcc; ++m)
      __builtin_amdgcn_raw_buffer_store_b128(o_lds[wave][o_slot(m * kRPI + orow, oblk)], u.o,
                                             o_at(u, m), 0, kStream);
  };

  // Software pipeline (see the file comment).  wA holds the weight tile of
  // the unit being computed; with double buffering a changed tile for the
  // next unit is loaded into wB one unit ahead and copied into wA before
  // that unit computes.  The input and prior-output loads run kAhead units
  // ahead: two for the rank <= 16 kernels on contiguous rows (a stage is 12
  // registers there, and with few units per workgroup the second unit in
  // flight hides more of the memory latency: llama7b-like q_proj 8.57 ->
  // 8.04 us), one otherwise (measured slower with two).
  constexpr bool kDoubleW = kSteps <= SGMV_DOUBLE_W_MAX_KSTEPS;
  constexpr int kAhead = KS == 0 && !GATHER ? 2 : 1;
  u32x4 wA[4][kSteps], wB[4][kDoubleW ? kSteps : 1];
  Stage<XD, OD, KS> sA, sB, sC;

  FastUnit cur = next_unit();
  load_w(wA, cur);
  int w_tile = cur.tile;
  int32_t w_a = cur.a;
  bool w_pending = false;
  load_stage(sA, cur);
  // With kAhead = 2, the next unit is decoded and its loads issued here.
  bool have_nxt = false;
  FastUnit nxt = cur;
  if constexpr (kAhead == 2) {
    have_nxt = pos.next();
    if (have_nxt) nxt = next_unit();
    load_stage(sB, nxt);
  }

  // One step: publish the current unit's input tile to LDS buffer `buf`,
  // issue the loads of the unit kAhead ahead (s_new), then compute and
  // store the current unit.  Without a next unit the loads repeat the last
  // one's, so every step issues the same memory instructions.  The LDS
  // buffers alternate; the barrier in publish_x also orders every wave's
  // reads of a buffer before the next write to it.
  auto step = [&](Stage<XD, OD, KS>& s_cur, Stage<XD, OD, KS>& s_new, int buf)
                  __attribute__((always_inline)) -> bool {
    publish_x(s_cur, buf);
    if constexpr (kDoubleW) {
      if (w_pending) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int ks = 0; ks < kSteps; ++ks) wA[s][ks] = wB[s][ks];
        w_pending = false;
      }
    }
    if constexpr (kAhead == 1) {
      have_nxt = pos.next();
      nxt = cur;
      if (have_nxt) nxt = next_unit();
    }
    // the weight tile of the next unit
    const bool wswitch = nxt.tile != w_tile || nxt.a != w_a;
    if constexpr (kDoubleW) {
      if (wswitch) {
        load_w(wB, nxt);
        w_pending = true;
        w_tile = nxt.tile;
        w_a = nxt.a;
      }
    }
    bool more2 = false;
    FastUnit nxt2 = nxt;
    if constexpr (kAhead == 2) {
      more2 = have_nxt && pos.next();
      if (more2) nxt2 = next_unit();
    }
    load_stage(s_new, nxt2);
    // Keep the ahead loads in front of this unit's waits and arithmetic.
    __builtin_amdgcn_sched_barrier(0);
    compute_store(s_cur, wA, cur, buf);
    if constexpr (!kDoubleW) {
      if (wswitch) {
        load_w(wA, nxt);
        w_tile = nxt.tile;
        w_a = nxt.a;
      }
    }
    if (!have_nxt) return false;
    cur = nxt;
    if constexpr (kAhead == 2) {
      nxt = nxt2;
      have_nxt = more2;
    }
    return true;
  };
  if constexpr (kAhead == 2) {
    // stages rotate A -> B -> C (KS = 0: no LDS input buffers)
    while (step(sA, sC, 0) && step(sB, sA, 0) && step(sC, sB, 0)) {
    }
  } else {
    while (step(sA, sB, 0) && step(sB, sA, 1)) {
    }
  }
}

// ---------------------------------------------------------------------------
// Generic kernel: any shape, stride, alignment and rank.
// ---------------------------------------------------------------------------

template <int XD, int WD, int OD, bool ADD>
__global__ __launch_bounds__(kThreads) void expand_generic(const Params p) {
  prefetch_params(p);
  extern __shared__ __align__(16) int32_t lds[];  // segment table, 4 * batches + 1 words
  __shared__ int32_t wave_total[kWaves];
  const SegTable tab = seg_table(lds, p.batches);
  const int32_t RT = build_tile_table(p, tab, wave_total);
  const uint32_t U = (uint32_t)RT * (uint32_t)p.total_tiles;
  if (U == 0) return;
  uint32_t u_begin, u_end;
  unit_range(p, U, &u_begin, &u_end);
  if (u_begin >= u_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int j = lane & 15;
  const int K = p.K;

  Cursor pos(p, tab, RT, u_begin);
  for (uint32_t u = u_begin;;) {
    const Unit un = pos.decode(wave, j);
    const SliceDesc& S = p.s[un.si];
    if (un.col0 < S.n) {
      const bool vec_x = S.flags & kVecX;
      const bool vec_w = S.flags & kVecW;
      const bool vec_o = S.flags & kVecOut;
      f32x4 acc[4];
      int64_t ocol[2];
      int ocnt[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t c = un.col0 + 32 * q + 8 * g;
        ocol[q] = un.t * p.out_stride + S.offset + c;
        ocnt[q] = un.row_ok ? clamp8(S.n - c) : 0;
        float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if constexpr (ADD) {
          u32x4 raw[raw_vecs<OD>()];
          load_any8<OD>(p.out, ocol[q], ocnt[q], vec_o, raw);
          out_values<OD>(raw, v);
        }
        acc[2 * q] = f32x4{v[0], v[1], v[2], v[3]};
        acc[2 * q + 1] = f32x4{v[4], v[5], v[6], v[7]};
      }
      // Rank in chunks of 32: lane group g holds rank block k0 + 8g.
      for (int k0 = 0; k0 < K; k0 += 32) {
        const int kb = k0 + 8 * g;
        u32x4 xraw[raw_vecs<XD>()];
        load_any8<XD>(S.x, un.t * S.x_stride + kb, un.row_ok ? clamp8(K - kb) : 0, vec_x,
                      xraw);
        const u32x4 xo = x_operand<XD, WD>(xraw);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int64_t n = weight_row(un.col0, s, j);
          u32x4 w;
          load_any8<WD>(S.w, (un.a * S.n + n) * K + kb, n < S.n ? clamp8(K - kb) : 0, vec_w,
                        &w);
          acc[s] = mfma<WD>(w, xo, acc[s]);
        }
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float v[8] = {acc[2 * q][0], acc[2 * q][1], acc[2 * q][2], acc[2 * q][3],
                            acc[2 * q + 1][0], acc[2 * q + 1][1], acc[2 * q + 1][2],
                            acc[2 * q + 1][3]};
        store_any8<OD>(p.out, ocol[q], ocnt[q], vec_o, v);
      }
    }
    if (++u == u_end) break;
    pos.advance();
  }
}

// ---------------------------------------------------------------------------
// Kernel tables.
// ---------------------------------------------------------------------------

template <int XD, int WD, int OD, int KS>
const void* fast_entry(bool add, bool gather) {
  if (gather)
    return add ? reinterpret_cast<const void*>(&expand_fast<XD, WD, OD, true, KS, true>)
               : reinterpret_cast<const void*>(&expand_fast<XD, WD, OD, false, KS, true>);
  return add ? reinterpret_cast<const void*>(&expand_fast<XD, WD, OD, true, KS, false>)
             : reinterpret_cast<const void*>(&expand_fast<XD, WD, OD, false, KS, false>);
}

template <int XD, int WD, int KS>
const void* fast_by_out(int od, bool add, bool gather) {
  switch (od) {
    case F16: return fast_entry<XD, WD, F16, KS>(add, gather);
    case BF16: return fast_entry<XD, WD, BF16, KS>(add, gather);
    case F32: return fast_entry<XD, WD, F32, KS>(add, gather);
    default: return nullptr;
  }
}

template <int KS>
const void* fast_table(int xd, int wd, int od, bool add, bool gather) {
  if (wd == BF16 && xd == BF16) return fast_by_out<BF16, BF16, KS>(od, add, gather);
  if (wd == BF16 && xd == F32) return fast_by_out<F32, BF16, KS>(od, add, gather);
  if (wd == F16 && xd == F16) return fast_by_out<F16, F16, KS>(od, add, gather);
  if (wd == F16 && xd == F32) return fast_by_out<F32, F16, KS>(od, add, gather);
  return nullptr;
}

}  // namespace dev
}  // namespace sgmv

// sgmv_shrink.h -- gfx950 device code for the LoRA-A projection (shrink),
// the step that produces SGMV expand-slice's inputs (included by the shrink
// kernel translation units; internal to libsgmv).
//
// Operation: the wiki page "Implementation: Predibase Lorax SGMV Expand
// Slice Kernel" (I/O Contract, Inputs; Usage Examples) describes the
// expand's inputs as the low-rank activations of the LoRA A projection,
// (total_tokens, rank), packed across sequences.  For segment b with adapter
// a = idx[b] in [0, lora_num) and each row t of the segment,
//     y_s[t][k] = scale * sum_h x[t][h] * A_s[a][k][h],   k in [0, K),
// for every slice s (lora_A stack A_s (L, K, H), output y_s (T, K)).  Rows of
// other segments are not written.  float32 inputs are rounded to the weight
// dtype first, as in the expand.
//
// Design.  The projection reads every input row once and writes a row of K
// values, so it is bound by reading x (and, with many adapters and short
// segments, by reading the lora_A stacks).  Per work unit -- a 16-row tile of
// one segment -- the four wavefronts of a workgroup split the hidden
// dimension into four contiguous quarters, each wave streams its quarter of
// the 16 input rows and of every lora_A row the slices need, and the partial
// sums are added through LDS at the end of the unit.  The slices share the
// input tile: their lora_A rows are just more K rows (k tiles) of one
// contraction, so a fused QKV projection reads x once.
//
// The contraction is y^T = A . x^T on the matrix cores
// (v_mfma_f32_16x16x32_{bf16,f16}): 16 lora_A rows are the A operand, the 16
// tokens of the tile the B operand, 32 hidden elements per instruction; lane
// group g holds the 8-element block 8 g of each 32-wide step, so one load
// instruction reads 64 contiguous bytes of each of 16 rows.  Each lane ends
// with 4 consecutive k of one token per k tile.  Loads go through buffer
// resources bounded by the tile's valid rows and the slice's K rows, so rows
// past the segment and k past K read zero and store nothing; hidden blocks
// past H take an offset outside every resource.  The step loop is double
// buffered in blocks of shrink_block_steps() steps, every block issuing the
// same load instructions (blocks past the wave's quarter read nothing), so
// the compiler waits for one block with a nonzero vmcnt.
#pragma once

#include "sgmv_device.h"

namespace sgmv {
namespace dev {

// This workgroup's contiguous range of the U units, the grid's XCD-aware
// remap as in the expand (each XCD owns one contiguous eighth).
__device__ __forceinline__ void shrink_units(const ShrinkParams& p, uint32_t U, uint32_t* begin,
                                             uint32_t* end) {
  unit_range(p, U, begin, end);
}

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

template <int XD, int KTT, int RT>
struct ShrinkBlock {
  static constexpr int kSteps = shrink_block_steps(XD, KTT, RT);
  u32x4 x[kSteps][RT][raw_vecs<XD>()];
  u32x4 a[kSteps][KTT];
};

// KTT: 16-row k tiles over all slices (a power of two >= the slices' total;
// tiles past it are dead: they read zero and store nothing).  RT: 16-row
// token tiles per unit.
template <int XD, int WD, int OD, int KTT, int RT>
__global__ __launch_bounds__(kThreads) void shrink_fast(const ShrinkParams p) {
  using Block = ShrinkBlock<XD, KTT, RT>;
  constexpr int kB = Block::kSteps;
  constexpr int kFrags = RT * KTT;
  constexpr int kRound = kFrags < 8 ? kFrags : 8;  // fragments added per LDS round
  constexpr int xb = XD == F32 ? 4 : 2;
  constexpr int ob = OD == F32 ? 4 : 2;
  prefetch_params(p);
  extern __shared__ __align__(16) int32_t lds[];  // segment table, 4 * batches + 1 words
  __shared__ int32_t wave_total[kWaves];
  __shared__ f32x4 red[kWaves][kRound][64];
  const SegTable tab = seg_table(lds, p.batches);
  const int32_t U = build_tile_table(p, tab, wave_total, kTileRows * RT);
  if (U == 0) return;
  uint32_t u, u_end;
  shrink_units(p, (uint32_t)U, &u, &u_end);
  if (u >= u_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int g = lane >> 4;  // lane group: hidden block 8 g of a step / k rows 4 g.. of a tile
  const int j = lane & 15;  // token of a tile / lora_A row of a k tile
  const int32_t H = p.H;
  const int32_t K = p.K;
  const int32_t kt_n = p.k_tiles;
  const uint32_t xrb = (uint32_t)p.x_row_bytes;  // 16 RT rows span < 2 GiB (host)
  const int32_t s_beg = wave * p.wave_steps;
  const int32_t s_end = s_beg + p.wave_steps;
  // lane parts of the load offsets: row j, hidden block 8 g
  const uint32_t x_lane = (uint32_t)j * xrb + (uint32_t)(8 * g * xb);
  const uint32_t a_lane = (uint32_t)j * (uint32_t)H * 2u + (uint32_t)(16 * g);

  int b = last_at_most(tab.tile_start, p.batches + 1, (int32_t)u);
  for (; u < u_end; ++u) {
    while (uniform(tab.tile_start[b + 1]) <= (int32_t)u) ++b;
    const int32_t row0 =
        uniform(tab.seg_row[b]) + ((int32_t)u - uniform(tab.tile_start[b])) * (kTileRows * RT);
    const int32_t left = uniform(tab.seg_end[b]) - row0;
    const int32_t rows = left < kTileRows * RT ? left : kTileRows * RT;
    const int64_t a = uniform(tab.seg_lora[b]);
    const rsrc_t xr = make_rsrc(static_cast<const char*>(p.x) + (int64_t)row0 * p.x_row_bytes,
                                (int64_t)rows * p.x_row_bytes);
    // k tile i: slice i / kt_n, rows 16 (i % kt_n) .. of A_s[a]
    auto a_rsrc = [&](int i) __attribute__((always_inline)) -> rsrc_t {
      const int si = i / kt_n;
      const int kt = i - si * kt_n;
      if (si >= p.num_slices) return make_rsrc(p.x, 0);
      const int32_t kr = K - 16 * kt < 16 ? K - 16 * kt : 16;
      return make_rsrc(static_cast<const char*>(p.s[si].a) + (a * K + 16 * kt) * H * 2,
                       (int64_t)kr * H * 2);
    };

    auto load_block = [&](Block& blk, int32_t s0) __attribute__((always_inline)) {
#pragma unroll
      for (int st = 0; st < kB; ++st) {
        const int32_t step = s0 + st;
        const bool ok = step < s_end && 32 * step + 8 * g < H;
#pragma unroll
        for (int r = 0; r < RT; ++r)
          buf_load8<XD>(xr, ok ? x_lane + (uint32_t)r * 16u * xrb + (uint32_t)(32 * step * xb)
                               : kOut,
                        blk.x[st][r]);
#pragma unroll
        for (int i = 0; i < KTT; ++i)
          buf_load8<WD>(a_rsrc(i), ok ? a_lane + (uint32_t)(64 * step) : kOut, &blk.a[st][i]);
      }
    };

    f32x4 acc[RT][KTT];
#pragma unroll
    for (int r = 0; r < RT; ++r)
#pragma unroll
      for (int i = 0; i < KTT; ++i) acc[r][i] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute_block = [&](const Block& blk) __attribute__((always_inline)) {
#pragma unroll
      for (int st = 0; st < kB; ++st)
#pragma unroll
        for (int r = 0; r < RT; ++r) {
          const u32x4 xo = x_operand<XD, WD>(blk.x[st][r]);
#pragma unroll
          for (int i = 0; i < KTT; ++i) acc[r][i] = mfma<WD>(blk.a[st][i], xo, acc[r][i]);
        }
    };

    // The wave's steps [s_beg, s_end) (a multiple of 2 kB), two blocks per
    // iteration; the last iteration's third load lies past s_end.
    Block b0, b1;
    load_block(b0, s_beg);
    for (int32_t s = s_beg; s < s_end; s += 2 * kB) {
      load_block(b1, s + kB);
      compute_block(b0);
      load_block(b0, s + 2 * kB);
      compute_block(b1);
    }

    // Add the four waves' partial sums through LDS, kRound fragments at a
    // time; wave w finishes fragments w, w + 4, ...  The first barrier of a
    // round also orders the previous round's (or unit's) reads before the
    // writes.
#pragma unroll
    for (int f0 = 0; f0 < kFrags; f0 += kRound) {
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kRound; ++q)
        if (f0 + q < kFrags) red[wave][q][lane] = acc[(f0 + q) / KTT][(f0 + q) % KTT];
      __syncthreads();
#pragma unroll
      for (int q = 0; q < kRound; ++q) {
        const int f = f0 + q;
        if (f >= kFrags || (q & (kWaves - 1)) != wave) continue;
        const int r = f / KTT, i = f % KTT;
        const int si = i / kt_n;
        if (si >= p.num_slices) continue;
        const int kt = i - si * kt_n;
        f32x4 v = red[0][q][lane];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) v += red[w][q][lane];
        v *= p.scale;
        const ShrinkSliceDesc& S = p.s[si];
        const rsrc_t orc = make_rsrc(static_cast<char*>(S.out) + (int64_t)row0 * S.out_row_bytes,
                                     (int64_t)rows * S.out_row_bytes);
        const int32_t k = 16 * kt + 4 * g;
        const uint32_t off =
            k < K ? (uint32_t)(16 * r + j) * (uint32_t)S.out_row_bytes + (uint32_t)(k * ob) : kOut;
        store4<OD>(orc, off, v);
      }
    }
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

template <int XD, int WD, int KTT>
const void* shrink_by_out(int od) {
  switch (od) {
    case F16: return reinterpret_cast<const void*>(&shrink_fast<XD, WD, F16, KTT, 1>);
    case BF16: return reinterpret_cast<const void*>(&shrink_fast<XD, WD, BF16, KTT, 1>);
    case F32: return reinterpret_cast<const void*>(&shrink_fast<XD, WD, F32, KTT, 1>);
    default: return nullptr;
  }
}

template <int KTT>
const void* shrink_table(int xd, int wd, int od) {
  if (wd == BF16 && xd == BF16) return shrink_by_out<BF16, BF16, KTT>(od);
  if (wd == BF16 && xd == F32) return shrink_by_out<F32, BF16, KTT>(od);
  if (wd == F16 && xd == F16) return shrink_by_out<F16, F16, KTT>(od);
  if (wd == F16 && xd == F32) return shrink_by_out<F32, F16, KTT>(od);
  return nullptr;
}

}  // namespace dev
}  // namespace sgmv

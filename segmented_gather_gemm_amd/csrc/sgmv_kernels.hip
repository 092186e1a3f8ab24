// sgmv_kernels.hip -- gfx950 kernels for SGMV expand-slice.
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
//    table of row-tile prefix sums -- the device-side scheduler.  Index -1
//    segments and segments outside [0, T) get no tiles.
//  * Work unit = (column tile of 256 output columns, 16-row tile of one
//    segment).  Units are ordered column-tile-major, so consecutive units of
//    a workgroup walk down the rows of a segment under one column tile and
//    the adapter's weight tile stays in registers across all of them.
//    Workgroups take equal contiguous unit ranges; workgroup ids are
//    remapped so that each XCD (ids are dealt round-robin to the 8 XCDs)
//    owns one contiguous eighth of the range, i.e. its own column tiles and
//    hence its own slice of every adapter's weights in its L2.
//  * Each of the 4 wavefronts owns 64 of the 256 columns.  The contraction
//    runs on the matrix cores as C^T = W . X^T with v_mfma_f32_16x16x32_
//    {bf16,f16}: the weight rows are the MFMA rows (A operand, stationary in
//    VGPRs), the 16 tokens of the tile are the MFMA columns (B operand).
//    Weight rows are assigned to MFMA rows so that every lane ends up holding
//    8 consecutive output columns of one token: the epilogue then reads the
//    prior output and writes the result with 16-byte accesses, 64 contiguous
//    bytes per token per instruction.
//  * The rank dimension is permuted consistently in both operands so each
//    lane loads one contiguous run of its token's input row.
//  * fp32 accumulation; with add_inputs the prior output seeds the
//    accumulator, so the result is rounded once (v_cvt_pk_{bf16,f16}_f32,
//    nearest even).  float32 inputs are rounded to the weight dtype first.
//  * Ragged edges (rank not a multiple of 8, slice width not a multiple of
//    64, unaligned offsets or strides) take element-wise paths; nothing
//    outside the output window or the active rows is read-modified-written.
#include "sgmv_launch.h"

namespace sgmv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { F16 = 0, BF16 = 1, F32 = 2 };

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// D = A . B + C on 16x16 fp32, A 16x32 and B 32x16 of the weight dtype.
template <int WD>
__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (WD == BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two floats -> one packed pair of 16-bit values, round to nearest even.
template <int D>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  if constexpr (D == BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}

// One 16-bit value (low half of h) -> float, exact.
template <int D>
__device__ __forceinline__ float widen(uint32_t h) {
  if constexpr (D == BF16)
    return __uint_as_float(h << 16);
  else
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ int clamp8(int64_t v) {
  return v <= 0 ? 0 : (v >= 8 ? 8 : (int)v);
}

// Eight consecutive elements of an XD matrix starting at element `e`, as a
// packed 16-bit operand of dtype WD.  `cnt` (0..8) leading elements are
// real, the rest read as zero.  `vec`: the block is 16-byte aligned.
template <int XD, int WD>
__device__ __forceinline__ u32x4 load8(const void* base, int64_t e, int cnt, bool vec) {
  u32x4 r;
  if constexpr (XD == F32) {
    const float* p = static_cast<const float*>(base) + e;
    float v[8];
    if (vec && cnt == 8) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p);
      const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
      v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
      v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = i < cnt ? p[i] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack2<WD>(v[2 * i], v[2 * i + 1]);
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + e;
    if (vec && cnt == 8) {
      r = *reinterpret_cast<const u32x4*>(p);
    } else {
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) h[i] = i < cnt ? (uint32_t)p[i] : 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = h[2 * i] | (h[2 * i + 1] << 16);
    }
  }
  return r;
}

// Eight consecutive output elements (first `cnt` real) -> floats.
template <int OD>
__device__ __forceinline__ void load_out8(const void* base, int64_t e, int cnt, bool vec,
                                          float* v) {
  if constexpr (OD == F32) {
    const float* p = static_cast<const float*>(base) + e;
    if (vec && cnt == 8) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(p);
      const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
      v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
      v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = i < cnt ? p[i] : 0.0f;
    }
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + e;
    if (vec && cnt == 8) {
      const u32x4 r = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = widen<OD>(r[i] & 0xFFFFu);
        v[2 * i + 1] = widen<OD>(r[i] >> 16);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = i < cnt ? widen<OD>(p[i]) : 0.0f;
    }
  }
}

// Round eight floats to the output dtype and store the first `cnt`.
template <int OD>
__device__ __forceinline__ void store_out8(void* base, int64_t e, int cnt, bool vec,
                                           const float* v) {
  if constexpr (OD == F32) {
    float* p = static_cast<float*>(base) + e;
    if (vec && cnt == 8) {
      *reinterpret_cast<f32x4*>(p) = f32x4{v[0], v[1], v[2], v[3]};
      *reinterpret_cast<f32x4*>(p + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < cnt) p[i] = v[i];
    }
  } else {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack2<OD>(v[2 * i], v[2 * i + 1]);
    uint16_t* p = static_cast<uint16_t*>(base) + e;
    if (vec && cnt == 8) {
      *reinterpret_cast<u32x4*>(p) = r;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < cnt) p[i] = (uint16_t)(i & 1 ? r[i / 2] >> 16 : r[i / 2] & 0xFFFFu);
    }
  }
}

// Largest b in [0, n) with table[b] <= key (table non-decreasing, table[0] = 0).
__device__ __forceinline__ int last_at_most(const int32_t* table, int n, int64_t key) {
  int lo = 0, hi = n;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uniform(table[mid]) <= key) lo = mid; else hi = mid;
  }
  return lo;
}

__device__ __forceinline__ int slice_of(const Params& p, int tile) {
  int si = 0;
  while (si + 1 < p.num_slices && p.s[si + 1].tile_begin <= tile) ++si;
  return si;
}

template <int XD, int WD, int OD, bool ADD, int KS>
__global__ __launch_bounds__(kThreads) void expand_kernel(const Params p) {
  extern __shared__ int32_t tile_start[];  // [batches + 1] row-tile prefix sums
  __shared__ int32_t wave_total[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // ---- 1. Segment scheduler: row tiles per active segment, exclusive scan.
  int32_t carry = 0;
  for (int base = 0; base < p.batches; base += kThreads) {
    const int b = base + tid;
    int32_t tiles = 0;
    if (b < p.batches) {
      const int64_t st = p.start[b], ln = p.lens[b], a = p.idx[b];
      if (a >= 0 && a < p.L && ln > 0 && st >= 0 && st <= p.T - ln)
        tiles = (int32_t)((ln + kTileRows - 1) / kTileRows);
    }
    int32_t incl = tiles;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) wave_total[wave] = incl;
    __syncthreads();
    int32_t before = carry, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const int32_t s = wave_total[w];
      before += w < wave ? s : 0;
      all += s;
    }
    if (b < p.batches) tile_start[b] = before + incl - tiles;
    carry += all;
    __syncthreads();
  }
  if (tid == 0) tile_start[p.batches] = carry;
  __syncthreads();

  // ---- 2. This workgroup's contiguous range of work units.
  const int64_t RT = uniform(carry);
  const int64_t U = RT * p.total_tiles;
  if (U == 0) return;
  const int bid = blockIdx.x;
  const int lw = (p.grid >= 16 && (p.grid & 7) == 0) ? (bid & 7) * (p.grid >> 3) + (bid >> 3)
                                                      : bid;
  const int64_t u_begin = U * lw / p.grid;
  const int64_t u_end = U * (lw + 1) / p.grid;
  if (u_begin >= u_end) return;

  const int g = lane >> 4;   // lane group: rank sub-block / column group
  const int j = lane & 15;   // token of the tile / MFMA row of the A operand
  const int K = p.K;
  const bool add = ADD;

  int tile = (int)(u_begin / RT);
  int64_t rt = u_begin - (int64_t)tile * RT;
  int b = last_at_most(tile_start, p.batches + 1, rt);
  while (uniform(tile_start[b + 1]) <= rt) ++b;  // skip empty segments
  int si = slice_of(p, tile);

  u32x4 wreg[4][KS];
  int w_tile = -1;
  int64_t w_adapter = -1;

  for (int64_t u = u_begin;;) {
    const SliceDesc& S = p.s[si];
    const int64_t col0 = (int64_t)(tile - S.tile_begin) * kTileCols + wave * kWaveCols;
    if (col0 < S.n) {
      const int64_t seg_start = p.start[b];
      const int64_t seg_len = p.lens[b];
      const int64_t a = p.idx[b];
      const int64_t r0 = (rt - uniform(tile_start[b])) * kTileRows;
      const bool vec_x = S.flags & kVecX;
      const bool vec_w = S.flags & kVecW;
      const bool vec_o = S.flags & kVecOut;

      // Weight tile: MFMA row i = j of subtile s = 2q + h holds weight row
      // n = col0 + 32q + 8(i/4) + 4h + i%4, so the accumulator rows a lane
      // group holds are 8 consecutive output columns.
      if (tile != w_tile || a != w_adapter) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int64_t n = col0 + 32 * (s >> 1) + 8 * (j >> 2) + 4 * (s & 1) + (j & 3);
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int kb = (g * KS + ks) * 8;
            const int cnt = n < S.n ? clamp8(K - kb) : 0;
            wreg[s][ks] = load8<WD, WD>(S.w, (a * S.n + n) * K + kb, cnt, vec_w);
          }
        }
        w_tile = tile;
        w_adapter = a;
      }

      // Input rows: lane (g, j) holds rank block g*KS + ks of token j.
      const int64_t row = r0 + j;
      const bool valid = row < seg_len;
      const int64_t t = seg_start + row;
      u32x4 xreg[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int kb = (g * KS + ks) * 8;
        xreg[ks] = load8<XD, WD>(S.x, t * S.x_stride + kb, valid ? clamp8(K - kb) : 0, vec_x);
      }

      // Accumulators, seeded with the prior output when accumulating.
      f32x4 acc[4];
      int64_t ocol[2];
      int ocnt[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int64_t c = col0 + 32 * q + 8 * g;
        ocol[q] = t * p.out_stride + S.offset + c;
        ocnt[q] = valid ? clamp8(S.n - c) : 0;
        float v[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (add) load_out8<OD>(p.out, ocol[q], ocnt[q], vec_o, v);
        acc[2 * q] = f32x4{v[0], v[1], v[2], v[3]};
        acc[2 * q + 1] = f32x4{v[4], v[5], v[6], v[7]};
      }

#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) acc[s] = mfma<WD>(wreg[s][ks], xreg[ks], acc[s]);

#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const float v[8] = {acc[2 * q][0], acc[2 * q][1], acc[2 * q][2], acc[2 * q][3],
                            acc[2 * q + 1][0], acc[2 * q + 1][1], acc[2 * q + 1][2],
                            acc[2 * q + 1][3]};
        store_out8<OD>(p.out, ocol[q], ocnt[q], vec_o, v);
      }
    }

    if (++u == u_end) break;
    if (++rt == RT) {
      rt = 0;
      ++tile;
      b = 0;
      si = slice_of(p, tile);
    }
    while (uniform(tile_start[b + 1]) <= rt) ++b;
  }
}

template <int XD, int WD, int OD, bool ADD>
const void* by_ksteps(int ks) {
  switch (ks) {
    case 1: return reinterpret_cast<const void*>(&expand_kernel<XD, WD, OD, ADD, 1>);
    case 2: return reinterpret_cast<const void*>(&expand_kernel<XD, WD, OD, ADD, 2>);
    case 4: return reinterpret_cast<const void*>(&expand_kernel<XD, WD, OD, ADD, 4>);
    case 8: return reinterpret_cast<const void*>(&expand_kernel<XD, WD, OD, ADD, 8>);
    default: return nullptr;
  }
}

template <int XD, int WD, int OD>
const void* by_add(bool add, int ks) {
  return add ? by_ksteps<XD, WD, OD, true>(ks) : by_ksteps<XD, WD, OD, false>(ks);
}

template <int XD, int WD>
const void* by_out(int od, bool add, int ks) {
  switch (od) {
    case F16: return by_add<XD, WD, F16>(add, ks);
    case BF16: return by_add<XD, WD, BF16>(add, ks);
    case F32: return by_add<XD, WD, F32>(add, ks);
    default: return nullptr;
  }
}

template <int WD>
const void* by_input(int xd, int od, bool add, int ks) {
  if (xd == WD) return by_out<WD, WD>(od, add, ks);
  if (xd == F32) return by_out<F32, WD>(od, add, ks);
  return nullptr;
}

}  // namespace

const void* kernel_for(const Variant& v) {
  if (v.wd == BF16) return by_input<BF16>(v.xd, v.od, v.add, v.ksteps);
  if (v.wd == F16) return by_input<F16>(v.xd, v.od, v.add, v.ksteps);
  return nullptr;
}

hipError_t launch(const void* kernel, const Params& p, int grid, size_t lds_bytes,
                  hipStream_t stream) {
  void* args[] = {const_cast<Params*>(&p)};
  return hipLaunchKernel(kernel, dim3(grid), dim3(kThreads), args, lds_bytes, stream);
}

}  // namespace sgmv

// sgmv_common.h -- gfx950 device helpers shared by the expand kernels
// (sgmv_device.h) and the LoRA-A projection kernels (sgmv_shrink.h):
// vector types, the MFMA wrapper, 16-bit packing, element-wise and buffer
// loads and stores, and the device-side segment scheduler (segment table
// in LDS, unit ranges).  Internal to libsgmv.
#pragma once

#include "sgmv_launch.h"
#include "sgmv_limits.h"

namespace sgmv {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { F16 = 0, BF16 = 1, F32 = 2 };

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

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

template <int D>
constexpr int raw_vecs() { return D == F32 ? 2 : 1; }

// Eight consecutive elements of dtype D at element `e` with 16-byte loads
// (one for 16-bit types, two for float32); the block must be aligned.
template <int D>
__device__ __forceinline__ void load_vec8(const void* base, int64_t e, u32x4* dst) {
  const uint32_t* p = reinterpret_cast<const uint32_t*>(static_cast<const char*>(base) +
                                                        e * (D == F32 ? 4 : 2));
  dst[0] = *reinterpret_cast<const u32x4*>(p);
  if constexpr (D == F32) dst[1] = *reinterpret_cast<const u32x4*>(p + 4);
}

// Eight consecutive elements of dtype D at element `e`, the first `cnt`
// (0..8) real and the rest zero; vector loads when `vec` (aligned) and the
// block is whole, element loads otherwise.
template <int D>
__device__ __forceinline__ void load_any8(const void* base, int64_t e, int cnt, bool vec,
                                          u32x4* dst) {
  if (vec && cnt == 8) {
    load_vec8<D>(base, e, dst);
    return;
  }
  if constexpr (D == F32) {
    const uint32_t* p = static_cast<const uint32_t*>(base) + e;
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = i < cnt ? p[i] : 0u;
    dst[0] = u32x4{v[0], v[1], v[2], v[3]};
    dst[1] = u32x4{v[4], v[5], v[6], v[7]};
  } else {
    const uint16_t* p = static_cast<const uint16_t*>(base) + e;
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = i < cnt ? (uint32_t)p[i] : 0u;
    dst[0] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                   h[6] | (h[7] << 16)};
  }
}

// Raw input block -> packed 16-bit MFMA operand of the weight dtype (float32
// inputs are rounded to nearest even here).
template <int XD, int WD>
__device__ __forceinline__ u32x4 x_operand(const u32x4* raw) {
  if constexpr (XD == F32) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      r[2 * i] = pack2<WD>(__uint_as_float(raw[i][0]), __uint_as_float(raw[i][1]));
      r[2 * i + 1] = pack2<WD>(__uint_as_float(raw[i][2]), __uint_as_float(raw[i][3]));
    }
    return r;
  } else {
    return raw[0];
  }
}

// Raw output block -> eight floats (exact).
template <int OD>
__device__ __forceinline__ void out_values(const u32x4* raw, float* v) {
  if constexpr (OD == F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(raw[0][i]);
      v[4 + i] = __uint_as_float(raw[1][i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = widen<OD>(raw[0][i] & 0xFFFFu);
      v[2 * i + 1] = widen<OD>(raw[0][i] >> 16);
    }
  }
}

// Eight floats -> raw output block (rounded to the output dtype).
template <int OD>
__device__ __forceinline__ void out_pack(const float* v, u32x4* raw) {
  if constexpr (OD == F32) {
    raw[0] = u32x4{__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                   __float_as_uint(v[3])};
    raw[1] = u32x4{__float_as_uint(v[4]), __float_as_uint(v[5]), __float_as_uint(v[6]),
                   __float_as_uint(v[7])};
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) raw[0][i] = pack2<OD>(v[2 * i], v[2 * i + 1]);
  }
}

template <int OD>
__device__ __forceinline__ void store_vec8(void* base, int64_t e, const u32x4* raw) {
  uint32_t* p = reinterpret_cast<uint32_t*>(static_cast<char*>(base) + e * (OD == F32 ? 4 : 2));
  *reinterpret_cast<u32x4*>(p) = raw[0];
  if constexpr (OD == F32) *reinterpret_cast<u32x4*>(p + 4) = raw[1];
}

// Store the first `cnt` of eight rounded output values (element-wise unless
// the block is whole and aligned).
template <int OD>
__device__ __forceinline__ void store_any8(void* base, int64_t e, int cnt, bool vec,
                                           const float* v) {
  u32x4 raw[raw_vecs<OD>()];
  out_pack<OD>(v, raw);
  if (vec && cnt == 8) {
    store_vec8<OD>(base, e, raw);
    return;
  }
  if constexpr (OD == F32) {
    float* p = static_cast<float*>(base) + e;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < cnt) p[i] = v[i];
  } else {
    uint16_t* p = static_cast<uint16_t*>(base) + e;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (i < cnt) p[i] = (uint16_t)(i & 1 ? raw[0][i / 2] >> 16 : raw[0][i / 2] & 0xFFFFu);
  }
}

// ---------------------------------------------------------------------------
// Scheduler.
// ---------------------------------------------------------------------------

// Inclusive prefix sum over the 64 lanes of a wave through DPP (VALU
// operands routed across lanes, no LDS round trip): shifts by 1, 2, 4 and 8
// within each 16-lane row, then lane 15 of each row added into the next row
// (rows 1 and 3) and lane 31 into rows 2 and 3.  Lanes a shift or broadcast
// does not reach add the `old` operand, 0.
__device__ __forceinline__ int32_t wave_inclusive_sum(int32_t v) {
  constexpr int kRowShr = 0x110, kRowBcast15 = 0x142, kRowBcast31 = 0x143;
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 1, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 2, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 4, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowShr + 8, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowBcast15, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, kRowBcast31, 0xc, 0xf, false);
  return v;
}

// Segment table in LDS, filled by build_tile_table, one slot per segment
// (slot order: see build_tile_table):
//   tile_start[0..batches]  exclusive prefix sum of row tiles per slot
//   seg_row[b], seg_end[b]  first row and one-past-last row of slot b's segment
//   seg_lora[b]             its adapter index
// A segment is active (gets tiles) when its index lies in [0, lora_num), its
// length is positive and it lies inside [0, T).
struct SegTable {
  int32_t* tile_start;
  int32_t* seg_row;
  int32_t* seg_end;
  int32_t* seg_lora;
};

// Kernel arguments live in memory and the compiler fetches each scalar on
// first use, so the scheduler's chain of uses would pay one dependent round
// trip per field.  Touch every 64-byte line of the argument block at kernel
// entry so all of them are fetched together; later reads hit the scalar
// cache.
template <typename P>
__device__ __forceinline__ void prefetch_params(const P& p) {
  const uint32_t* w = reinterpret_cast<const uint32_t*>(&p);
  constexpr int kLast = (int)(sizeof(P) / 4) - 1;
  static_assert(sizeof(P) <= 576, "touch list below covers 9 lines");
  asm volatile("" ::"s"(w[0]), "s"(w[16 < kLast ? 16 : kLast]), "s"(w[32 < kLast ? 32 : kLast]),
               "s"(w[48 < kLast ? 48 : kLast]), "s"(w[64 < kLast ? 64 : kLast]),
               "s"(w[80 < kLast ? 80 : kLast]), "s"(w[96 < kLast ? 96 : kLast]),
               "s"(w[112 < kLast ? 112 : kLast]), "s"(w[128 < kLast ? 128 : kLast]),
               "s"(w[kLast]));
}

__device__ __forceinline__ SegTable seg_table(int32_t* lds, int batches) {
  SegTable t;
  t.tile_start = lds;
  t.seg_row = lds + (batches + 1);
  t.seg_end = t.seg_row + batches;
  t.seg_lora = t.seg_end + batches;
  return t;
}

// Exclusive prefix sum of v[0 .. n) in place (all NT threads take part, v
// written before the call is visible to them; wave_total holds NT / 64
// words); returns the total (wave-uniform).
template <int NT>
__device__ __forceinline__ int32_t block_exclusive_scan(int32_t* v, int n, int32_t* wave_total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t carry = 0;
  for (int base = 0; base < n; base += NT) {
    const int i = base + tid;
    const int32_t x = i < n ? v[i] : 0;
    const int32_t incl = wave_inclusive_sum(x);
    if (lane == 63) wave_total[wave] = incl;
    __syncthreads();
    int32_t before = carry, all = 0;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
      const int32_t s = wave_total[w];
      before += w < wave ? s : 0;
      all += s;
    }
    if (i < n) v[i] = before + incl - x;
    carry += all;
    __syncthreads();
  }
  return uniform(carry);
}

// Table of a per-token call whose row tiles gather the tokens of one adapter
// (up to 16 per tile, in token order): the adapter of every token (-1: none
// or out of range), each adapter's token count and the exclusive prefix of
// its tile counts.  B + 2 L + 1 words of LDS.
struct GatherTable {
  int32_t* tok_a;    // [B]
  int32_t* a_tiles;  // [L + 1] first row tile of adapter a; a_tiles[L] = row tiles
  int32_t* a_count;  // [L] tokens of adapter a
};

__device__ __forceinline__ GatherTable gather_table(int32_t* lds, int batches, int adapters) {
  GatherTable t;
  t.tok_a = lds;
  t.a_tiles = lds + batches;
  t.a_count = t.a_tiles + adapters + 1;
  return t;
}

// Fill the gathered table (all kThreads threads take part): count each
// adapter's tokens (LDS atomics: the counts do not depend on their order),
// then the tile prefix.  Returns the number of row tiles (wave-uniform).
template <typename P>
__device__ __forceinline__ int32_t build_gather_table(const P& p, const GatherTable& gt,
                                                      int32_t* wave_total) {
  const int tid = threadIdx.x;
  const int B = p.batches, L = p.L;
  for (int a = tid; a < L; a += kThreads) gt.a_count[a] = 0;
  __syncthreads();
  for (int b = tid; b < B; b += kThreads) {
    const int64_t a = p.idx[b];
    const bool active = a >= 0 && a < L && b < p.T;
    gt.tok_a[b] = active ? (int32_t)a : -1;
    if (active) atomicAdd(&gt.a_count[a], 1);
  }
  __syncthreads();
  for (int a = tid; a < L; a += kThreads) gt.a_tiles[a] = (gt.a_count[a] + kTileRows - 1) / kTileRows;
  __syncthreads();
  const int32_t total = block_exclusive_scan<kThreads>(gt.a_tiles, L, wave_total);
  if (tid == 0) gt.a_tiles[L] = total;
  __syncthreads();
  return total;
}


// Fill the table (all NT threads of the workgroup take part; wave_total
// holds NT / 64 words) with row tiles of `tile_rows` rows; returns the total
// number of row tiles (wave-uniform).  P: the kernel's argument block
// (segment metadata fields as in Params).
template <int NT = kThreads, typename P>
__device__ __forceinline__ int32_t build_tile_table(const P& p, const SegTable& tab,
                                                    int32_t* wave_total,
                                                    int32_t tile_rows = kTileRows) {
  constexpr int kThreads = NT;         // shadows the default block size below
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int B = p.batches;
  // Segment b: its row range, adapter and row-tile count (0 when inactive).
  auto read_segment = [&](int b, int32_t* row, int32_t* end, int32_t* a32,
                          int32_t* tiles) __attribute__((always_inline)) {
    const int64_t st = p.per_token ? b : p.start[b];
    const int64_t ln = p.per_token ? 1 : p.lens[b];
    const int64_t a = p.idx[b];
    const bool active = a >= 0 && a < p.L && ln > 0 && st >= 0 && st <= p.T - ln;
    *row = active ? (int32_t)st : 0;
    *end = active ? (int32_t)(st + ln) : 0;
    *a32 = active ? (int32_t)a : -1;
    *tiles = active ? (int32_t)((ln + tile_rows - 1) / tile_rows) : 0;
  };
  // First pass: table slot of every segment; tile_start[slot] temporarily
  // holds the segment's tile count.
  // With p.sort_slots the table lists segments in order of (adapter, index),
  // inactive ones last, so that segments sharing an adapter are adjacent in
  // the walk and its weight tiles are reused instead of re-read; otherwise
  // in index order.  Every workgroup computes the same order.
  if (p.sort_slots && B <= kSortMaxBatches) {
    // Unique 32-bit keys (adapter << 9 | index; inactive: 1 << 31 | index;
    // the host orders only when adapters < 2^22 and batches <= 512) in
    // tile_start[0 .. B), padded to a multiple of 4 with 0xffffffff, which
    // is never below a key.  The padding spills into seg_row's first words,
    // which are written only after the ranks are taken.
    constexpr int kPer = (kSortMaxBatches + kThreads - 1) / kThreads;
    int32_t row[kPer], end[kPer], a32[kPer], tiles[kPer];
    uint32_t key[kPer];
    uint32_t* keys = reinterpret_cast<uint32_t*>(tab.tile_start);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = tid + i * kThreads;
      key[i] = 0xffffffffu;
      if (b < B) {
        read_segment(b, &row[i], &end[i], &a32[i], &tiles[i]);
        key[i] = (a32[i] < 0 ? 0x80000000u : (uint32_t)a32[i] << 9) | (uint32_t)b;
        keys[b] = key[i];
      }
    }
    const int B4 = (B + 3) & ~3;
    if (tid < B4 - B) keys[B + tid] = 0xffffffffu;
    __syncthreads();
    // Slot of segment b = number of keys below its key: four keys per
    // 16-byte LDS read (a broadcast: every lane reads the same address) and a
    // compare and an add per key.
    uint32_t slot[kPer];
#pragma unroll
    for (int i = 0; i < kPer; ++i) slot[i] = 0;
    const uint4* keys4 = reinterpret_cast<const uint4*>(keys);
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (i * kThreads < B) {  // uniform: whether any segment has this i
#pragma unroll 4
        for (int c4 = 0; c4 < B4 / 4; ++c4) {
          const uint4 k4 = keys4[c4];
          slot[i] += (k4.x < key[i]) + (k4.y < key[i]) + (k4.z < key[i]) + (k4.w < key[i]);
        }
      }
    }
    __syncthreads();  // every key read before the slots are written
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int b = tid + i * kThreads;
      if (b < B) {
        tab.tile_start[slot[i]] = tiles[i];
        tab.seg_row[slot[i]] = row[i];
        tab.seg_end[slot[i]] = end[i];
        tab.seg_lora[slot[i]] = a32[i] < 0 ? 0 : a32[i];
      }
    }
  } else if (B <= 64) {
    // Index order, every segment in one lane of wave 0: the tile counts are
    // scanned in registers and the table is complete after one barrier.
    if (wave == 0) {
      int32_t row = 0, end = 0, a32 = -1, tiles = 0;
      if (lane < B) read_segment(lane, &row, &end, &a32, &tiles);
      const int32_t incl = wave_inclusive_sum(tiles);
      if (lane < B) {
        tab.tile_start[lane] = incl - tiles;
        tab.seg_row[lane] = row;
        tab.seg_end[lane] = end;
        tab.seg_lora[lane] = a32 < 0 ? 0 : a32;
      }
      if (lane == 63) tab.tile_start[B] = incl;  // lanes >= B hold no tiles
    }
    __syncthreads();
    return uniform(tab.tile_start[B]);
  } else {
    for (int b = tid; b < B; b += kThreads) {
      int32_t row, end, a32, tiles;
      read_segment(b, &row, &end, &a32, &tiles);
      tab.tile_start[b] = tiles;
      tab.seg_row[b] = row;
      tab.seg_end[b] = end;
      tab.seg_lora[b] = a32 < 0 ? 0 : a32;
    }
  }
  __syncthreads();
  // Second pass: exclusive prefix sum of the tile counts over table slots.
  const int32_t total = block_exclusive_scan<kThreads>(tab.tile_start, B, wave_total);
  if (tid == 0) tab.tile_start[B] = total;
  __syncthreads();
  return total;
}

// The scheduler's arithmetic is 32-bit: unit counts, unit indices and
// row-tile counts are below 2^31 (the host refuses larger problems), and
// 64-bit division is a long scalar sequence that every wave of a compute
// unit would queue for on the shared scalar ALU.

// This workgroup's contiguous range [begin, end) of the U units
// (limits::unit_span: balanced shares per XCD while every unit can have a
// compute unit of its own, XCD-major contiguous ranges otherwise).
template <typename P>
__device__ __forceinline__ void unit_range(const P& p, uint32_t U, uint32_t* begin,
                                           uint32_t* end) {
  const limits::UnitSpan s = limits::unit_span(U, (uint32_t)p.grid, (uint32_t)p.cus, blockIdx.x);
  *begin = s.begin;
  *end = s.end;
}

// Largest b in [0, n) with table[b] <= key (table non-decreasing, table[0] =
// 0).  Wave-uniform; called with every lane of the wave active.  Up to 64
// entries: one LDS read per lane and a ballot (the entries <= key are a
// prefix of the table), else a binary search.
__device__ __forceinline__ int last_at_most(const int32_t* table, int n, int32_t key) {
  if (n <= 64) {
    const int l = threadIdx.x & 63;
    const bool le = l < n && table[l] <= key;
    return __builtin_popcountll(__ballot(le)) - 1;
  }
  int lo = 0, hi = n;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (uniform(table[mid]) <= key) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// Buffer resources.
// ---------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer resource over [base, base + bytes): a 16-byte access at an
// offset past `bytes` reads zero and writes nothing.  The fourth word selects
// 32-bit data format, as untyped buffer accesses require on gfx9.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int32_t n = bytes <= 0 ? 0 : (int32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

// Lane offset that lies past every resource this kernel builds (the host
// only picks the fast kernel when 16 rows of inputs or output span < 2 GiB).
constexpr uint32_t kOut = 0x80000000u;

// Cache policy of a load: 0 is the default; kStreamLoad (non-temporal) for
// data that is read once.
constexpr int kStreamLoad = 0x2;  // nt

template <int D, int POLICY = 0>
__device__ __forceinline__ void buf_load8(rsrc_t r, uint32_t off, u32x4* dst) {
  dst[0] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, POLICY));
  if constexpr (D == F32)
    dst[1] = __builtin_bit_cast(
        u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16), 0, POLICY));
}

// Cache policy of a store: 0 is the default; kStream (non-temporal at device
// scope) marks lines that are written once and not read again, so they do not
// displace reused weight and input lines from L2.
constexpr int kStream = 0x12;  // nt | sc1

template <int D, int POLICY = 0>
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, const u32x4* src) {
  __builtin_amdgcn_raw_buffer_store_b128(src[0], r, (int)off, 0, POLICY);
  if constexpr (D == F32)
    __builtin_amdgcn_raw_buffer_store_b128(src[1], r, (int)(off + 16), 0, POLICY);
}

}  // namespace dev
}  // namespace sgmv

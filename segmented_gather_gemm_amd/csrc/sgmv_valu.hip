// sgmv_valu.hip -- a vector-ALU form of the SGMV expand-slice for rank <= 32
// (internal to libsgmv): the same operation as the fast kernels
// (sgmv_device.h), with dot products on the vector ALU (v_dot2 with fp32
// accumulation) instead of the matrix cores.  It exists to measure the
// choice between the two on MI355X: the host takes it for rank <= 32 only
// when libsgmv is built with SGMV_EXPAND_VALU defined.
//
// Work unit = (256-column tile, 16-row tile of one segment), as in the other
// kernels, walked column tile by column tile (consecutive units of a
// workgroup run down the rows under one column tile, so the lora_B rows stay
// in registers).  Each of the 4 wavefronts owns 64 columns, one per lane:
// lane n holds lora_B[a][col0 + n][0 .. K) (K <= 32: up to 4 16-byte
// blocks).  The wave stages the unit's 16 input rows in its own LDS region
// (one 16-byte load per lane; float32 inputs rounded to the weight dtype on
// the way) and every lane reads each row back as a broadcast; each lane then
// computes its column of the 16 rows as chains of K / 2 v_dot2 steps seeded
// with the prior output (add_inputs), rounds once to the output dtype and
// stores it (2 or 4 bytes per lane and row: 128 or 256 contiguous bytes per
// row and wave).
#include "sgmv_device.h"

namespace sgmv {
namespace dev {

template <int WD>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (WD == BF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c,
                                  false);
}

template <int XD, int WD, int OD, bool ADD>
__global__ __launch_bounds__(kThreads) void expand_valu(const Params p) {
  constexpr int kMaxQ = 4;  // 16-byte blocks of a rank-32 row
  constexpr int xb = XD == F32 ? 4 : 2;
  constexpr int ob = OD == F32 ? 4 : 2;
  prefetch_params(p);
  extern __shared__ __align__(16) int32_t lds[];  // segment table, 4 * batches + 1 words
  __shared__ int32_t wave_total[kWaves];
  __shared__ u32x4 xs[kWaves][kTileRows * kMaxQ];  // each wave's input tile
  const SegTable tab = seg_table(lds, p.batches);
  const int32_t RT = build_tile_table(p, tab, wave_total);
  const uint32_t U = (uint32_t)RT * (uint32_t)p.total_tiles;
  if (U == 0) return;
  uint32_t u_begin, u_end;
  unit_range(p, U, &u_begin, &u_end);
  if (u_begin >= u_end) return;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);
  const int K = p.K;
  const int KQ = (K + 7) >> 3;  // 16-byte blocks of a row (K % 8 == 0 on this path)
  // input tile load: lane l reads block l % KQ of row l / KQ (lanes past the
  // tile's 16 KQ blocks read nothing)
  const int xr = lane / KQ, xq = lane % KQ;

  Cursor pos(p, tab, RT, u_begin);
  u32x4 w[kMaxQ];
  int w_tile = -1;
  int64_t w_a = -1;
  for (uint32_t u = u_begin;;) {
    const Unit un = pos.decode(wave, 0);
    const SliceDesc& S = p.s[un.si];
    const int64_t n_left = S.n - un.col0;
    const int32_t n_rem = n_left <= 0 ? 0 : (n_left > kWaveCols ? kWaveCols : (int32_t)n_left);
    const int64_t seg_end = uniform(tab.seg_end[pos.b]);
    const int64_t row0 = un.t;  // token 0 of the tile
    const int32_t rows = (int32_t)(seg_end - row0 < kTileRows ? seg_end - row0 : kTileRows);
    if (un.tile != w_tile || un.a != w_a) {
      const rsrc_t wr = make_rsrc(static_cast<const char*>(S.w) + (un.a * S.n + un.col0) * K * 2,
                                  (int64_t)n_rem * K * 2);
#pragma unroll
      for (int q = 0; q < kMaxQ; ++q)
        w[q] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             wr, q < KQ ? (uint32_t)(lane * K * 2 + 16 * q) : kOut,
                                             0, 0));
      w_tile = un.tile;
      w_a = un.a;
    }
    // the unit's input rows -> this wave's LDS tile (weight dtype)
    {
      const rsrc_t xrs = make_rsrc(static_cast<const char*>(S.x) + row0 * S.x_row_bytes,
                                   (int64_t)rows * S.x_row_bytes);
      u32x4 raw[raw_vecs<XD>()];
      buf_load8<XD>(xrs, xr < kTileRows ? (uint32_t)(xr * S.x_row_bytes + 8 * xq * xb) : kOut, raw);
      if (xr < kTileRows) xs[wave][xr * kMaxQ + xq] = x_operand<XD, WD>(raw);
    }
    // this lane's column: output bytes of row r at r * row_bytes + col_off
    const rsrc_t orc = make_rsrc(static_cast<char*>(p.out) + row0 * p.out_row_bytes,
                                 (int64_t)rows * p.out_row_bytes);
    const uint32_t col_off = lane < n_rem ? (uint32_t)((S.offset + un.col0 + lane) * ob) : kOut;
    float acc[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      acc[r] = 0.f;
      if constexpr (ADD) {
        const uint32_t off = col_off == kOut ? kOut : (uint32_t)(r * p.out_row_bytes) + col_off;
        if constexpr (OD == F32)
          acc[r] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(orc, (int)off, 0, 0));
        else
          acc[r] = widen<OD>(__builtin_amdgcn_raw_buffer_load_b16(orc, (int)off, 0, 0));
      }
    }
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
#pragma unroll
      for (int q = 0; q < kMaxQ; ++q) {
        if (q < KQ) {
          const u32x4 x = xs[wave][r * kMaxQ + q];  // broadcast: one address for the wave
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[r] = dot2<WD>(w[q][e], x[e], acc[r]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) {
      const uint32_t off = col_off == kOut ? kOut : (uint32_t)(r * p.out_row_bytes) + col_off;
      if constexpr (OD == F32)
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r]), orc, (int)off, 0, kStream);
      else
        __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(pack2<OD>(acc[r], 0.f) & 0xFFFFu), orc,
                                              (int)off, 0, kStream);
    }
    if (++u == u_end) break;
    pos.advance();
  }
}

template <int XD, int WD>
const void* valu_by_out(int od, bool add) {
  switch (od) {
    case F16: return add ? (const void*)&expand_valu<XD, WD, F16, true> : (const void*)&expand_valu<XD, WD, F16, false>;
    case BF16: return add ? (const void*)&expand_valu<XD, WD, BF16, true> : (const void*)&expand_valu<XD, WD, BF16, false>;
    case F32: return add ? (const void*)&expand_valu<XD, WD, F32, true> : (const void*)&expand_valu<XD, WD, F32, false>;
    default: return nullptr;
  }
}

}  // namespace dev

const void* valu_kernel(int xd, int wd, int od, bool add) {
  using namespace dev;
  if (wd == BF16 && xd == BF16) return valu_by_out<BF16, BF16>(od, add);
  if (wd == BF16 && xd == F32) return valu_by_out<F32, BF16>(od, add);
  if (wd == F16 && xd == F16) return valu_by_out<F16, F16>(od, add);
  if (wd == F16 && xd == F32) return valu_by_out<F32, F16>(od, add);
  return nullptr;
}

}  // namespace sgmv

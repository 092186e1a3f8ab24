// sgmv_fused_api.cpp -- libsgmv C entry point of the fused LoRA delta
// (sgmv_fused_shrink_expand): argument checks, kernel choice, grid sizing
// and launch.  No allocation, no synchronisation, no device-to-host
// traffic; the projected rows live in LDS only.
//
// The wiki page "Implementation: Predibase Lorax SGMV Expand Slice Kernel"
// describes the expand's inputs as the rank-sized activations of the A-side
// LoRA projection (I/O Contract, Inputs; Usage Examples) and motivates the
// slice kernel by a later fused operator over several slices in one launch
// (Description); this call is that projection and the expand of its result
// for the slices of a fused QKV or gate/up layer.
#include <stdint.h>

#include "sgmv.h"
#include "sgmv_fused_launch.h"
#include "sgmv_host.h"
#include "sgmv_limits.h"

namespace {

using namespace sgmv::host;
using sgmv::limits::next_pow2;
using sgmv::limits::shrink_fast_lora_a_fits;

const void* pick_fused_kernel(int xd, int wd, int od, bool add, int k16, int ns, bool split_h) {
  using namespace sgmv;
  switch (k16) {
    case 1: return fused_kernel_k1(xd, wd, od, add, ns, split_h);
    case 2: return fused_kernel_k2(xd, wd, od, add, ns, split_h);
    case 4: return fused_kernel_k4(xd, wd, od, add, ns, split_h);
    case 8: return fused_kernel_k8(xd, wd, od, add, ns, split_h);
    default: return nullptr;
  }
}

}  // namespace

extern "C" {

sgmv_status sgmv_fused_shrink_expand(sgmv_matrix inputs, const sgmv_fused_slice* slices,
                                     int num_slices, sgmv_matrix out,
                                     const int64_t* b_seq_start_loc, const int64_t* seq_lens,
                                     const int64_t* lora_indices, int64_t batches,
                                     int64_t max_seq_len, float scale, int add_inputs,
                                     hipStream_t stream) {
  using namespace sgmv;
  if (!slices) return fail(SGMV_ERR_INVALID_ARGUMENT, "slices pointer is null");
  if (num_slices < 1 || num_slices > SGMV_MAX_FUSED_SLICES)
    return fail(SGMV_ERR_INVALID_ARGUMENT, "num_slices must be in 1..%d, got %d",
                SGMV_MAX_FUSED_SLICES, num_slices);
  const sgmv_matrix& x = inputs;
  if (!known_dtype(x.dtype)) return fail(SGMV_ERR_INVALID_ARGUMENT, "unknown inputs dtype %d", x.dtype);
  if (!known_dtype(out.dtype)) return fail(SGMV_ERR_INVALID_ARGUMENT, "unknown output dtype %d", out.dtype);
  if (x.rows < 0 || x.cols < 1 || x.row_stride < x.cols)
    return fail(SGMV_ERR_INVALID_ARGUMENT,
                "inputs shape (%lld, %lld) with row stride %lld is invalid", (long long)x.rows,
                (long long)x.cols, (long long)x.row_stride);
  if (out.rows != x.rows || out.cols < 0 || out.row_stride < out.cols)
    return fail(SGMV_ERR_INVALID_ARGUMENT,
                "output (%lld, %lld) with row stride %lld must have the inputs' %lld rows",
                (long long)out.rows, (long long)out.cols, (long long)out.row_stride,
                (long long)x.rows);
  if (x.rows > INT32_MAX)
    return fail(SGMV_ERR_UNSUPPORTED, "more than 2^31-1 tokens (%lld)", (long long)x.rows);
  if (batches < 0) return fail(SGMV_ERR_INVALID_ARGUMENT, "batches must be >= 0");
  if (batches > SGMV_MAX_BATCHES)
    return fail(SGMV_ERR_UNSUPPORTED, "batches %lld exceeds %d", (long long)batches,
                SGMV_MAX_BATCHES);
  if (max_seq_len < 0) return fail(SGMV_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 0");

  const sgmv_fused_slice& s0 = slices[0];
  const int64_t K = s0.lora_a.rows, L = s0.lora_a.num, H = x.cols;
  for (int i = 0; i < num_slices; ++i) {
    const sgmv_fused_slice& s = slices[i];
    if (!known_dtype(s.lora_a.dtype) || !known_dtype(s.lora_b.dtype))
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: unknown dtype", i);
    if (s.lora_a.dtype == SGMV_F32 || s.lora_b.dtype != s.lora_a.dtype)
      return fail(SGMV_ERR_UNSUPPORTED,
                  "slice %d: lora_a and lora_b must share one 16-bit dtype", i);
    if (x.dtype != s.lora_a.dtype && x.dtype != SGMV_F32)
      return fail(SGMV_ERR_UNSUPPORTED,
                  "slice %d: inputs must have the weights' dtype or float32", i);
    if (s.lora_a.num < 0 || s.lora_a.rows < 1 || s.lora_a.cols != H)
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: lora_a must be (lora_num, rank, %lld)", i, (long long)H);
    if (s.lora_b.num != s.lora_a.num || s.lora_b.cols != s.lora_a.rows || s.lora_b.rows < 0)
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: lora_b must be (lora_num, slice_size, rank) with lora_a's "
                  "lora_num and rank", i);
    if (s.slice_offset < 0 || s.slice_offset > out.cols - s.lora_b.rows)
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: window [%lld, %lld) is outside the %lld output columns", i,
                  (long long)s.slice_offset, (long long)(s.slice_offset + s.lora_b.rows),
                  (long long)out.cols);
    if (i > 0 && (s.lora_a.rows != K || s.lora_a.num != L || s.lora_a.dtype != s0.lora_a.dtype))
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: rank, lora_num and dtypes must match slice 0", i);
    for (int q = 0; q < i; ++q) {
      const sgmv_fused_slice& o = slices[q];
      if (s.lora_b.rows > 0 && o.lora_b.rows > 0 &&
          s.slice_offset < o.slice_offset + o.lora_b.rows &&
          o.slice_offset < s.slice_offset + s.lora_b.rows)
        return fail(SGMV_ERR_INVALID_ARGUMENT, "slices %d and %d overlap", q, i);
    }
  }
  if (L > INT32_MAX) return fail(SGMV_ERR_UNSUPPORTED, "lora_num exceeds 2^31-1");
  int64_t total_tiles = 0;
  for (int i = 0; i < num_slices; ++i)
    total_tiles += (slices[i].lora_b.rows + kTileCols - 1) / kTileCols;
  if (batches == 0 || x.rows == 0 || total_tiles == 0) {
    g_error.clear();
    return SGMV_OK;  // nothing to do
  }
  if (!x.data || !out.data) return fail(SGMV_ERR_INVALID_ARGUMENT, "null data pointer");
  if (!b_seq_start_loc || !seq_lens || !lora_indices)
    return fail(SGMV_ERR_INVALID_ARGUMENT, "segment metadata pointer is null");
  for (int i = 0; i < num_slices; ++i)
    if (L > 0 && (!slices[i].lora_a.data || (slices[i].lora_b.rows > 0 && !slices[i].lora_b.data)))
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: null data pointer", i);

  // The kernels' shapes: rank a multiple of 8 up to 128 with k16 * slices <=
  // 16 (k16 = next power of two of ceil(rank / 16)), hidden a multiple of 8,
  // slice widths multiples of 8, 16-byte aligned data, rows and windows, and
  // 32-bit buffer offsets over 64 rows of inputs and output and over one
  // adapter's lora_A rows.
  const int64_t xb = elem_bytes(x.dtype), ob = elem_bytes(out.dtype);
  const int64_t k16 = next_pow2((K + 15) / 16);
  bool ok = K % 8 == 0 && K <= 128 && k16 * num_slices <= 16 && H % 8 == 0 &&
            H < (int64_t(1) << 26) && shrink_fast_lora_a_fits(K, H) && aligned16(x.data) &&
            aligned16(out.data) && (x.row_stride * xb) % 16 == 0 &&
            (out.row_stride * ob) % 16 == 0 &&
            kFusedTokens * x.row_stride * xb < (int64_t(1) << 31) &&
            kFusedTokens * out.row_stride * ob < (int64_t(1) << 31);
  for (int i = 0; i < num_slices && ok; ++i) {
    const sgmv_fused_slice& s = slices[i];
    ok = aligned16(s.lora_a.data) && aligned16(s.lora_b.data) && s.lora_b.rows % 8 == 0 &&
         (s.slice_offset * ob) % 16 == 0;
  }
  if (!ok)
    return fail(SGMV_ERR_UNSUPPORTED,
                "the fused call takes rank %% 8 == 0 up to 128 (16 * next_pow2(ceil(rank / 16)) "
                "* slices <= 256), hidden %% 8 == 0, slice widths %% 8 == 0 and 16-byte "
                "aligned rows and windows; run sgmv_shrink_multi_slice and "
                "sgmv_expand_multi_slice instead");
  if (total_tiles > INT32_MAX) return fail(SGMV_ERR_UNSUPPORTED, "output window too wide");

  FusedParams p{};
  p.x = x.data;
  p.start = b_seq_start_loc;
  p.lens = seq_lens;
  p.idx = lora_indices;
  p.x_row_bytes = x.row_stride * xb;
  p.T = x.rows;
  p.H = (int32_t)H;
  p.batches = (int32_t)batches;
  p.L = (int32_t)L;
  p.K = (int32_t)K;
  p.num_slices = num_slices;
  p.scale = scale;
  p.total_tiles = (int32_t)total_tiles;
  p.out = out.data;
  p.out_row_bytes = out.row_stride * ob;
  // Units of one adapter next to each other: each XCD then works through a
  // few adapters and finds their lora_B rows in its L2.
  p.sort_slots = batches <= kSortMaxBatches && L <= (1 << 22);
  int32_t tile_begin = 0;
  for (int i = 0; i < num_slices; ++i) {
    const sgmv_fused_slice& s = slices[i];
    FusedSliceDesc& d = p.s[i];
    d.a = s.lora_a.data;
    d.w = s.lora_b.data;
    d.n = s.lora_b.rows;
    d.offset = s.slice_offset;
    d.tile_begin = tile_begin;
    tile_begin += (int32_t)((s.lora_b.rows + kTileCols - 1) / kTileCols);
  }
  // The projection's form follows the workspace-free shrink's rule (so the
  // result equals that shrink followed by the expand, bit for bit):
  // split-T from shrink_split_t_min_units(k16) units of 64 tokens, split-H
  // below.
  const bool split_h =
      (x.rows + kFusedTokens - 1) / kFusedTokens < shrink_split_t_min_units((int)k16);
  const void* kernel = pick_fused_kernel(x.dtype, s0.lora_a.dtype, out.dtype, add_inputs != 0,
                                         (int)k16, num_slices, split_h);
  if (!kernel) return fail(SGMV_ERR_UNSUPPORTED, "no fused kernel for this dtype combination");
  const int64_t steps = (H + 31) / 32;
  if (split_h) {
    // each wave takes a quarter of the hidden steps; loop positions in whole
    // turns of the ring (as the split-H shrink)
    const int64_t per_wave = (steps + kWaves - 1) / kWaves;
    const int64_t turn = shrink_ring(shrink_block_loads_h(x.dtype, (int)k16 * num_slices)) *
                         shrink_block_steps_h(x.dtype, (int)k16 * num_slices);
    p.steps = (int32_t)((per_wave + turn - 1) / turn * turn);
  } else {
    // every wave runs all hidden steps; loop positions in whole turns of the
    // ring of blocks (as the split-T shrink)
    const int64_t turn = shrink_ring(shrink_block_loads_t(x.dtype, (int)k16, num_slices)) *
                         shrink_block_steps_t((int)k16 * num_slices);
    p.steps = (int32_t)((steps + turn - 1) / turn * turn);
  }

  const size_t lds = (size_t)(4 * batches + 1) * sizeof(int32_t);
  int capacity = 0, cus = 0;
  hipError_t e = device_capacity(kernel, lds, &capacity, &cus);
  if (e != hipSuccess)
    return fail(SGMV_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  if (capacity < 1)
    return fail(SGMV_ERR_UNSUPPORTED,
                "%lld segments: the fused kernel's segment table and staging buffers exceed a "
                "compute unit's LDS; run sgmv_shrink_multi_slice and sgmv_expand_multi_slice "
                "instead", (long long)batches);
  // Units are tiles of active segments: at most ceil(T / rows) + min(batches,
  // T).  Split-T: one per workgroup while they fit on the chip.  Split-H:
  // work items (a unit and a column group) up to about one per compute unit
  // (the device sizes the groups from the actual unit count).
  const int64_t rows = split_h ? kTileRows : kFusedTokens;
  const int64_t units = (x.rows + rows - 1) / rows + (batches < x.rows ? batches : x.rows);
  // One item per compute unit (measured on fused_q_proj / fused_decode_qkv:
  // two per compute unit double the projections a compute unit runs and
  // lose 20-25%; one column group per unit loses 30% on fused_q_proj).
  const int64_t want = split_h && units < cus ? cus : units;
  int64_t grid = want < capacity ? want : capacity;
  if (grid > 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  p.grid = (int32_t)grid;
  // At most the grid: whenever a unit has several column groups, every
  // workgroup then takes at most one item.
  p.item_target = (int32_t)(grid < cus ? grid : cus);
  p.cus = cus;
  void* args[] = {&p};
  e = hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(kThreads), args, lds, stream);
  if (e != hipSuccess) return fail(SGMV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_error.clear();
  return SGMV_OK;
}

}  // extern "C"

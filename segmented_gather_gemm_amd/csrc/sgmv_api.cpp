// sgmv_api.cpp -- libsgmv C entry points: argument checks, kernel variant
// choice, grid sizing and launch.  No allocation, no synchronisation, no
// device-to-host traffic: the segment metadata stays on the device and the
// kernels schedule themselves from it.
//
// The checks follow the I/O Contract of the wiki page "Implementation:
// Predibase Lorax SGMV Expand Slice Kernel": inputs (total_tokens, rank);
// lora_b (lora_num, slice_size, rank) float16/bfloat16; output
// (total_tokens, full_hidden_size); slice_size equal to lora_b's row count.
#include <stdint.h>

#include "sgmv.h"
#include "sgmv_host.h"
#include "sgmv_launch.h"

namespace {

using namespace sgmv::host;

// Row tiles (16 rows each) per band of the fast kernels' walk: each XCD
// covers its column group band by band, so a band's input rows and weight
// tiles are re-read from its L2 rather than from memory.
#ifndef SGMV_BAND_TILES
#define SGMV_BAND_TILES 64
#endif
constexpr int32_t kBandTiles = SGMV_BAND_TILES;

// Units per chunk of the fast kernels' strided assignment: a workgroup keeps
// its weight tile in registers over a chunk, and the workgroups of an XCD
// stay within about (workgroups per XCD) chunks of each other in the walk.
#ifndef SGMV_CHUNK_UNITS
#define SGMV_CHUNK_UNITS 32
#endif
constexpr int32_t kChunkUnits = SGMV_CHUNK_UNITS;

// Smallest number of work units per workgroup the grid is sized for (from the
// host's upper bound on units; large problems run at full occupancy anyway).
#ifndef SGMV_UNITS_PER_WORKGROUP
#define SGMV_UNITS_PER_WORKGROUP 3
#endif
constexpr int64_t kUnitsPerWorkgroup = SGMV_UNITS_PER_WORKGROUP;
static_assert(sgmv::kGatherMaxTokens == SGMV_MAX_BATCHES, "every per-token call can gather");
static_assert(kChunkUnits >= 1 && kBandTiles % kChunkUnits == 0,
              "chunks must not straddle a column tile's run of a band");



int ksteps_for(int64_t rank) {
  if (rank <= 16) return 0;
  if (rank <= 32) return 1;
  if (rank <= 64) return 2;
  if (rank <= 128) return 4;
  return 8;  // rank <= SGMV_MAX_RANK
}

bool fast_rank(int64_t K) { return K % 8 == 0 && K <= SGMV_MAX_RANK; }

// The kernel for a call: a fast (pipelined) kernel when rank, slice widths
// and alignment allow it (`fast`), with gathered row tiles for `gather`
// (per-token calls only), else the generic one.
const void* pick_kernel(int xd, int wd, int od, bool add, int64_t K, bool fast, bool gather) {
  using namespace sgmv;
  if (fast) {
    switch (ksteps_for(K)) {
      case 0: return fast_kernel_ks0(xd, wd, od, add, gather);
      case 1: return fast_kernel_ks1(xd, wd, od, add, gather);
      case 2: return fast_kernel_ks2(xd, wd, od, add, gather);
      case 4: return fast_kernel_ks4(xd, wd, od, add, gather);
      default: return fast_kernel_ks8(xd, wd, od, add, gather);
    }
  }
  return generic_kernel(xd, wd, od, add);
}


// Checks shared by the entry points.  `slices` are host descriptors.  With
// `per_token` (the BGMV form) segment b is row b alone: start and lens are
// not used and batches = the number of rows.
sgmv_status check_and_launch(const sgmv_slice* slices, int num_slices, sgmv_matrix out,
                             const int64_t* start, const int64_t* lens, const int64_t* idx,
                             int64_t batches, int64_t max_seq_len, int add_inputs,
                             hipStream_t stream, bool per_token = false) {
  using namespace sgmv;
  if (num_slices < 1 || num_slices > SGMV_MAX_SLICES)
    return fail(SGMV_ERR_INVALID_ARGUMENT, "num_slices must be in 1..%d, got %d",
                SGMV_MAX_SLICES, num_slices);
  if (!known_dtype(out.dtype))
    return fail(SGMV_ERR_INVALID_ARGUMENT, "unknown output dtype %d", out.dtype);
  if (out.rows < 0 || out.cols < 0 || out.row_stride < out.cols)
    return fail(SGMV_ERR_INVALID_ARGUMENT,
                "output shape (%lld, %lld) with row stride %lld is invalid",
                (long long)out.rows, (long long)out.cols, (long long)out.row_stride);
  if (out.rows > INT32_MAX)
    return fail(SGMV_ERR_UNSUPPORTED, "more than 2^31-1 tokens (%lld)", (long long)out.rows);
  if (batches < 0) return fail(SGMV_ERR_INVALID_ARGUMENT, "batches must be >= 0");
  if (batches > SGMV_MAX_BATCHES)
    return fail(SGMV_ERR_UNSUPPORTED, "batches %lld exceeds %d", (long long)batches,
                SGMV_MAX_BATCHES);
  if (max_seq_len < 0) return fail(SGMV_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 0");

  const sgmv_slice& s0 = slices[0];
  const int64_t K = s0.inputs.cols;
  const int64_t L = s0.lora_b.num;
  for (int i = 0; i < num_slices; ++i) {
    const sgmv_slice& s = slices[i];
    if (!known_dtype(s.inputs.dtype) || !known_dtype(s.lora_b.dtype))
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: unknown dtype", i);
    if (s.lora_b.dtype == SGMV_F32)
      return fail(SGMV_ERR_UNSUPPORTED, "slice %d: lora_b must be float16 or bfloat16", i);
    if (s.inputs.dtype != s.lora_b.dtype && s.inputs.dtype != SGMV_F32)
      return fail(SGMV_ERR_UNSUPPORTED,
                  "slice %d: inputs must have lora_b's dtype or float32 (got %d with %d)", i,
                  s.inputs.dtype, s.lora_b.dtype);
    if (s.inputs.rows < 0 || s.inputs.cols < 1 || s.inputs.row_stride < s.inputs.cols)
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: inputs shape (%lld, %lld) with row stride %lld is invalid", i,
                  (long long)s.inputs.rows, (long long)s.inputs.cols,
                  (long long)s.inputs.row_stride);
    if (s.lora_b.num < 0 || s.lora_b.rows < 0 || s.lora_b.cols < 1)
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: lora_b shape is invalid", i);
    if (s.inputs.cols != s.lora_b.cols)
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: inputs rank %lld != lora_b rank %lld",
                  i, (long long)s.inputs.cols, (long long)s.lora_b.cols);
    if (s.lora_b.rows != s.slice_size)
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: slice_size %lld must equal lora_b.size(-2) = %lld", i,
                  (long long)s.slice_size, (long long)s.lora_b.rows);
    if (s.inputs.rows != out.rows)
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: inputs rows %lld != output rows %lld",
                  i, (long long)s.inputs.rows, (long long)out.rows);
    if (s.slice_offset < 0 || s.slice_size < 0 || s.slice_offset > out.cols - s.slice_size)
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: window [%lld, %lld) is outside the %lld output columns", i,
                  (long long)s.slice_offset, (long long)(s.slice_offset + s.slice_size),
                  (long long)out.cols);
    if (i > 0) {
      if (s.inputs.cols != K || s.lora_b.num != L || s.inputs.dtype != s0.inputs.dtype ||
          s.lora_b.dtype != s0.lora_b.dtype)
        return fail(SGMV_ERR_INVALID_ARGUMENT,
                    "slice %d: rank, lora_num and dtypes must match slice 0", i);
    }
    for (int j = 0; j < i; ++j) {
      const sgmv_slice& o = slices[j];
      if (s.slice_size > 0 && o.slice_size > 0 &&
          s.slice_offset < o.slice_offset + o.slice_size &&
          o.slice_offset < s.slice_offset + s.slice_size)
        return fail(SGMV_ERR_INVALID_ARGUMENT, "slices %d and %d overlap", j, i);
    }
  }
  if (K > INT32_MAX) return fail(SGMV_ERR_UNSUPPORTED, "rank exceeds 2^31-1");
  if (L > INT32_MAX) return fail(SGMV_ERR_UNSUPPORTED, "lora_num exceeds 2^31-1");

  int64_t total_tiles = 0;
  for (int i = 0; i < num_slices; ++i)
    total_tiles += (slices[i].slice_size + kTileCols - 1) / kTileCols;
  if (batches == 0 || out.rows == 0 || total_tiles == 0) {
    g_error.clear();
    return SGMV_OK;  // nothing to do
  }
  if (total_tiles > INT32_MAX) return fail(SGMV_ERR_UNSUPPORTED, "output window too wide");
  // Upper bound on work units from host-known sizes only: active segments are
  // disjoint inside [0, T), so row tiles <= ceil(T / 16) + min(batches, T).
  // The kernels' scheduler counts units in 32 bits.
  const int64_t row_tiles = (out.rows + kTileRows - 1) / kTileRows +
                            (batches < out.rows ? batches : out.rows);
  const int64_t units = row_tiles * total_tiles;
  if (units > INT32_MAX)
    return fail(SGMV_ERR_UNSUPPORTED, "more than 2^31-1 work units (16-row x 256-column tiles)");
  if (!out.data) return fail(SGMV_ERR_INVALID_ARGUMENT, "output data pointer is null");
  if ((!per_token && (!start || !lens)) || !idx)
    return fail(SGMV_ERR_INVALID_ARGUMENT, "segment metadata pointer is null");
  for (int i = 0; i < num_slices; ++i) {
    if (slices[i].slice_size == 0) continue;
    if (!slices[i].inputs.data || (!slices[i].lora_b.data && L > 0))
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: null data pointer", i);
  }

  Params p{};
  p.out = out.data;
  p.start = start;
  p.lens = lens;
  p.idx = idx;
  p.out_stride = out.row_stride;
  p.out_row_bytes = out.row_stride * elem_bytes(out.dtype);
  p.band_tiles = kBandTiles;
  p.chunk_units = kChunkUnits;
  p.per_token = per_token ? 1 : 0;
  p.T = out.rows;
  p.batches = (int32_t)batches;
  p.L = (int32_t)L;
  p.K = (int32_t)K;
  p.num_slices = num_slices;
  p.total_tiles = (int32_t)total_tiles;
  const int64_t ob = elem_bytes(out.dtype);
  int32_t tile_begin = 0;
  for (int i = 0; i < num_slices; ++i) {
    const sgmv_slice& s = slices[i];
    SliceDesc& d = p.s[i];
    d.x = s.inputs.data;
    d.w = s.lora_b.data;
    d.x_stride = s.inputs.row_stride;
    d.x_row_bytes = s.inputs.row_stride * elem_bytes(s.inputs.dtype);
    d.n = s.slice_size;
    d.offset = s.slice_offset;
    d.tile_begin = tile_begin;
    tile_begin += (int32_t)((s.slice_size + kTileCols - 1) / kTileCols);
    const int64_t xb = elem_bytes(s.inputs.dtype);
    d.flags = 0;
    if (aligned16(s.inputs.data) && (s.inputs.row_stride * xb) % 16 == 0 && K % 8 == 0)
      d.flags |= kVecX;
    if (aligned16(s.lora_b.data) && K % 8 == 0) d.flags |= kVecW;
    if (aligned16(out.data) && (out.row_stride * ob) % 16 == 0 && (s.slice_offset * ob) % 16 == 0)
      d.flags |= kVecOut;
  }

  // Fast kernels: whole 16-byte blocks everywhere, and 16 rows of inputs or
  // output spanning less than 2 GiB (their buffer offsets are 32-bit).
  bool fast_shapes = 16 * p.out_row_bytes < (int64_t(1) << 31);
  for (int i = 0; i < num_slices; ++i) {
    if (slices[i].slice_size == 0) continue;
    const int32_t need = kVecX | kVecW | kVecOut;
    if (slices[i].slice_size % 8 != 0 || (p.s[i].flags & need) != need ||
        16 * p.s[i].x_row_bytes >= (int64_t(1) << 31))
      fast_shapes = false;
  }
  const bool fast = fast_shapes && fast_rank(K);
  // Per-token calls on the fast kernels gather each adapter's tokens into
  // common row tiles (one weight tile and one MFMA pass for up to 16 tokens)
  // when they are few enough for the gathered table in LDS and T rows of the
  // inputs and of the output span less than 2 GiB (32-bit row offsets).
  // Otherwise per-token calls, calls of many segments and large calls order
  // the segment table by adapter (when it is cheap enough), so that
  // neighbours that share an adapter share its weight tiles.
  bool gather = fast && per_token && batches <= kGatherMaxTokens && L <= kGatherMaxAdapters &&
                out.rows * p.out_row_bytes < (int64_t(1) << 31);
  for (int i = 0; i < num_slices && gather; ++i)
    if (out.rows * p.s[i].x_row_bytes >= (int64_t(1) << 31)) gather = false;
  int64_t adapter_bytes = 0;  // one adapter's weights over all slices
  for (int i = 0; i < num_slices; ++i)
    adapter_bytes += slices[i].slice_size * K * elem_bytes(slices[i].lora_b.dtype);
  const bool large = units >= kSortMinUnits && adapter_bytes >= kSortMinAdapterBytes;
  const bool sort = !gather && (per_token || batches >= kSortMinBatches || large) &&
                    batches <= kSortMaxBatches && L <= (1 << 22);
  p.sort_slots = sort;
  p.gather = gather;
  const void* kernel =
      pick_kernel(s0.inputs.dtype, s0.lora_b.dtype, out.dtype, add_inputs != 0, K, fast, gather);
#ifdef SGMV_EXPAND_VALU
  if (fast && !gather && K <= 32)
    kernel = valu_kernel(s0.inputs.dtype, s0.lora_b.dtype, out.dtype, add_inputs != 0);
#endif
  if (!kernel) return fail(SGMV_ERR_UNSUPPORTED, "no kernel for this dtype combination");

  // segment table, or the gathered table
  const size_t lds =
      (size_t)(gather ? batches + 2 * L + 1 : 4 * batches + 1) * sizeof(int32_t);
  int capacity = 0, cus = 0;
  hipError_t e = device_capacity(kernel, lds, &capacity, &cus);
  if (e != hipSuccess)
    return fail(SGMV_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  // About kUnitsPerWorkgroup units per workgroup at least: a workgroup that
  // holds several units overlaps each one's loads with the previous one's
  // work, and idle workgroups still pay for the segment table.
  const int64_t want = (units + kUnitsPerWorkgroup - 1) / kUnitsPerWorkgroup;
  int64_t grid = want < capacity ? want : capacity;
  if (grid > 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  p.grid = (int32_t)grid;
  p.cus = cus;

  void* args[] = {&p};
  e = hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(kThreads), args, lds, stream);
  if (e != hipSuccess) return fail(SGMV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  g_error.clear();
  return SGMV_OK;
}

}  // namespace

extern "C" {

sgmv_status sgmv_expand_slice(sgmv_matrix inputs, sgmv_stack lora_b, sgmv_matrix out,
                              const int64_t* b_seq_start_loc, const int64_t* seq_lens,
                              const int64_t* lora_indices, int64_t batches,
                              int64_t max_seq_len, int64_t slice_offset, int64_t slice_size,
                              int add_inputs, hipStream_t stream) {
  sgmv_slice s;
  s.inputs = inputs;
  s.lora_b = lora_b;
  s.slice_offset = slice_offset;
  s.slice_size = slice_size;
  return check_and_launch(&s, 1, out, b_seq_start_loc, seq_lens, lora_indices, batches,
                          max_seq_len, add_inputs, stream);
}

sgmv_status sgmv_expand_multi_slice(const sgmv_slice* slices, int num_slices, sgmv_matrix out,
                                    const int64_t* b_seq_start_loc, const int64_t* seq_lens,
                                    const int64_t* lora_indices, int64_t batches,
                                    int64_t max_seq_len, int add_inputs, hipStream_t stream) {
  if (!slices) return fail(SGMV_ERR_INVALID_ARGUMENT, "slices pointer is null");
  return check_and_launch(slices, num_slices, out, b_seq_start_loc, seq_lens, lora_indices,
                          batches, max_seq_len, add_inputs, stream);
}

sgmv_status sgmv_bgmv_expand_slice(sgmv_matrix inputs, sgmv_stack lora_b, sgmv_matrix out,
                                   const int64_t* lora_indices, int64_t slice_offset,
                                   int64_t slice_size, int add_inputs, hipStream_t stream) {
  if (out.rows > SGMV_MAX_BATCHES)
    return fail(SGMV_ERR_UNSUPPORTED, "per-token calls take at most %d tokens, got %lld",
                SGMV_MAX_BATCHES, (long long)out.rows);
  sgmv_slice s;
  s.inputs = inputs;
  s.lora_b = lora_b;
  s.slice_offset = slice_offset;
  s.slice_size = slice_size;
  return check_and_launch(&s, 1, out, nullptr, nullptr, lora_indices, out.rows < 0 ? 0 : out.rows,
                          1, add_inputs, stream, true);
}

const char* sgmv_last_error(void) { return sgmv::host::g_error.c_str(); }

int sgmv_abi_version(void) { return SGMV_ABI_VERSION; }

}  // extern "C"

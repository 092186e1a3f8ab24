// sgmv_launch.h -- interface between the host entry points (sgmv_api.cpp)
// and the gfx950 kernels (sgmv_kernels.hip).  Internal to libsgmv.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sgmv {

constexpr int kMaxSlices = 8;
constexpr int kThreads = 256;          // 4 wavefronts of 64 lanes
constexpr int kWaves = kThreads / 64;
constexpr int kWaveCols = 64;          // output columns one wavefront owns per unit
constexpr int kTileCols = kWaves * kWaveCols;  // columns per work unit (256)
constexpr int kTileRows = 16;          // rows per work unit (one MFMA column block)

// Bits of SliceDesc::flags: 16-byte vector access is legal for ...
enum : int32_t {
  kVecX = 1,    // ... every 8-element block of an input row
  kVecW = 2,    // ... every 8-element block of a weight row
  kVecOut = 4,  // ... every 8-element column group of the output window
};

struct SliceDesc {
  const void* x;        // inputs (T, K), row stride x_stride elements
  const void* w;        // lora_b (L, N, K) contiguous
  int64_t x_stride;
  int64_t n;            // slice_size
  int64_t offset;       // slice_offset
  int32_t tile_begin;   // first global column-tile index of this slice
  int32_t flags;
};

struct Params {
  void* out;
  const int64_t* start;
  const int64_t* lens;
  const int64_t* idx;
  int64_t out_stride;   // elements
  int64_t T;            // rows of out (and of every inputs matrix)
  int32_t batches;
  int32_t L;            // lora_num
  int32_t K;            // rank
  int32_t num_slices;
  int32_t total_tiles;  // column tiles over all slices
  int32_t grid;         // workgroups launched
  SliceDesc s[kMaxSlices];
};

// Kernel variant: dtypes, accumulate flag and the number of 32-wide rank
// steps held in registers (K <= 32 * ksteps).
struct Variant {
  int xd, wd, od;
  bool add;
  int ksteps;
};

// Returns the kernel entry for a variant, or nullptr if none is built.
const void* kernel_for(const Variant& v);

// Launch `kernel` with `grid` workgroups of kThreads and `lds_bytes` of
// dynamic LDS.  Returns the HIP status of the launch.
hipError_t launch(const void* kernel, const Params& p, int grid, size_t lds_bytes,
                  hipStream_t stream);

}  // namespace sgmv

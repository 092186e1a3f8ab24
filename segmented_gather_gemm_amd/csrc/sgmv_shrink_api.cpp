// sgmv_shrink_api.cpp -- libsgmv C entry points of the LoRA-A projection
// (shrink): argument checks, kernel choice, grid sizing and launch.  No
// allocation, no synchronisation, no device-to-host traffic.
//
// The projection produces the expand's inputs, which the wiki page
// "Implementation: Predibase Lorax SGMV Expand Slice Kernel" (I/O Contract,
// Inputs; Usage Examples) describes as the low-rank activations of the LoRA
// A projection, (total_tokens, rank); lora_A is taken as (lora_num, rank,
// hidden), out-by-in like lora_B.
#include <stdint.h>

#include <map>
#include <mutex>

#include <hip/hip_runtime.h>

#include "sgmv.h"
#include "sgmv_host.h"
#include "sgmv_limits.h"
#include "sgmv_shrink_launch.h"

namespace {

using namespace sgmv::host;
using sgmv::limits::shrink_fast_lora_a_fits;

// Fast shrink kernel for k16 tiles of 16 rows per slice and ns slices.
const void* pick_shrink_kernel(int xd, int wd, int od, int k16, int ns, bool split_t) {
  using namespace sgmv;
  switch (k16) {
    case 1: return shrink_kernel_k1(xd, wd, od, ns, split_t);
    case 2: return shrink_kernel_k2(xd, wd, od, ns, split_t);
    case 4: return shrink_kernel_k4(xd, wd, od, ns, split_t);
    case 8: return shrink_kernel_k8(xd, wd, od, ns, split_t);
    default: return shrink_kernel_k16(xd, wd, od, ns, split_t);
  }
}

int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// With a workspace the split-T kernel cuts the units of small batches into
// hidden parts (limits::part_plan), and for ranks above 64 it then beats
// split-H from this many units (measured, 16-63 units of 64 tokens, hidden
// 4096-8192: rank 128 42 -> 25-36 us, rank 256 73 -> 26-34 us; ranks of 64
// and below gain little or lose, so they keep the threshold above).  The
// choice depends on the rank and the batch only, never on the slice count,
// so a multi-slice call and its single calls take the same kernel form.
#ifndef SGMV_SHRINK_SPLIT_T_MIN_UNITS_WIDE
#define SGMV_SHRINK_SPLIT_T_MIN_UNITS_WIDE 16
#endif

// One launch over slices [first, first + count) of `slices` (already checked).
sgmv_status shrink_launch(const sgmv_matrix& x, const sgmv_shrink_slice* slices, int first,
                          int count, const int64_t* start, const int64_t* lens,
                          const int64_t* idx, int64_t batches, float scale, bool fast,
                          bool split_t, void* workspace, hipStream_t stream) {
  using namespace sgmv;
  const sgmv_shrink_slice& s0 = slices[first];
  const int64_t K = s0.lora_a.rows;
  const int64_t H = x.cols;
  const int k16 = next_pow2((int)((K + 15) / 16));
  ShrinkParams p{};
  p.x = x.data;
  p.start = start;
  p.lens = lens;
  p.idx = idx;
  p.x_row_bytes = x.row_stride * elem_bytes(x.dtype);
  p.T = x.rows;
  p.H = (int32_t)H;
  p.batches = (int32_t)batches;
  p.L = (int32_t)s0.lora_a.num;
  p.K = (int32_t)K;
  p.num_slices = count;
  p.scale = scale;
  p.sort_slots = batches >= kSortMinBatches && batches <= kSortMaxBatches &&
                 s0.lora_a.num <= (1 << 22);
  for (int i = 0; i < count; ++i) {
    const sgmv_shrink_slice& s = slices[first + i];
    p.s[i].a = s.lora_a.data;
    p.s[i].out = s.out.data;
    p.s[i].out_row_bytes = s.out.row_stride * elem_bytes(s.out.dtype);
  }
  const void* kernel =
      fast ? pick_shrink_kernel(x.dtype, s0.lora_a.dtype, s0.out.dtype, k16, count, split_t)
           : shrink_generic_kernel(x.dtype, s0.lora_a.dtype, s0.out.dtype);
  if (!kernel) return fail(SGMV_ERR_UNSUPPORTED, "no shrink kernel for this dtype combination");
  const int64_t steps = (H + 31) / 32;  // 32-wide hidden steps
  if (fast && split_t) {
    // every wave runs all steps; loop positions in whole turns of the ring
    // of blocks
    const int64_t turn = shrink_ring(shrink_block_loads_t(x.dtype, k16, count)) *
                         shrink_block_steps_t(k16 * count);
    p.steps = (int32_t)((steps + turn - 1) / turn * turn);
  } else if (fast) {
    // each wave takes a quarter of the steps; loop positions in whole turns
    // of the ring
    const int64_t per_wave = (steps + kWaves - 1) / kWaves;
    const int64_t turn = shrink_ring(shrink_block_loads_h(x.dtype, k16 * count)) *
                         shrink_block_steps_h(x.dtype, k16 * count);
    p.steps = (int32_t)((per_wave + turn - 1) / turn * turn);
  }
  const size_t lds = (size_t)(4 * batches + 1) * sizeof(int32_t);
  int capacity = 0, cus = 0;
  hipError_t e = device_capacity(kernel, lds, &capacity, &cus);
  if (e != hipSuccess)
    return fail(SGMV_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  // Units are tiles of active segments: at most ceil(T / rows) + min(batches,
  // T) of them.  One per workgroup while they fit on the chip.
  const int64_t tile_rows = fast && split_t ? kShrinkTokensSplitT : kTileRows;
  const int64_t units =
      (x.rows + tile_rows - 1) / tile_rows + (batches < x.rows ? batches : x.rows);
  int64_t grid = units < capacity ? units : capacity;
  // With a workspace, split-T launches get a workgroup per compute unit at
  // least, and two when the batch may have more units than compute units,
  // so that the kernel can balance its units (limits::part_plan); the
  // choice depends only on the unit bound and the device, never on the
  // slices' kernel.
  if (fast && split_t && workspace) {
    const int64_t least = (units > cus ? 2 : 1) * (int64_t)cus;
    if (grid < least) grid = least;
  }
  if (grid > 8) grid -= grid % 8;
  if (grid < 1) grid = 1;
  p.grid = (int32_t)grid;
  p.cus = cus;
  p.ws = fast && split_t ? workspace : nullptr;
  void* args[] = {&p};
  e = hipLaunchKernel(kernel, dim3((unsigned)grid), dim3(kThreads), args, lds, stream);
  if (e != hipSuccess) return fail(SGMV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SGMV_OK;
}

// ---------------------------------------------------------------------------
// Allocation-free variant (sgmv_shrink_multi_slice_noalloc): the workspace
// is a static device array of the library, one copy per device, held until
// the process ends.
// ---------------------------------------------------------------------------

// Largest compute-unit count the static workspace covers (MI355X: 256).
constexpr int kNoAllocMaxCus = 320;
constexpr int64_t kNoAllocBytes = sgmv::limits::shrink_workspace_bytes(kNoAllocMaxCus);

// In host code `scratch` is a host-side stand-in, not a device address:
// only the address hipGetSymbolAddress gives (noalloc_workspace) may reach a
// kernel or a copy.
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch;  // device -> address of its copy of scratch

// The current device's copy of scratch, looked up on the first call on that
// device (with it current) and kept.
hipError_t noalloc_workspace(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    it = g_scratch.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

// Zero n part counters (a kernel, not a memset, so that graph capture records
// a kernel node).
__global__ void zero_counters(uint32_t* counters, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counters[i] = 0u;
}

// Clears the part counters at the start of `workspace` on `stream`.
sgmv_status clear_workspace_counters(void* workspace, hipStream_t stream) {
  int cus = 0;
  hipError_t e = device_compute_units(&cus);
  if (e != hipSuccess) return fail(SGMV_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  const int n = (int)(sgmv::limits::shrink_workspace_counter_bytes(cus) / 4);
  hipLaunchKernelGGL(zero_counters, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<uint32_t*>(workspace), n);
  e = hipGetLastError();
  if (e != hipSuccess) return fail(SGMV_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return SGMV_OK;
}

sgmv_status shrink_check_and_launch(sgmv_matrix x, const sgmv_shrink_slice* slices,
                                    int num_slices, const int64_t* start, const int64_t* lens,
                                    const int64_t* idx, int64_t batches, int64_t max_seq_len,
                                    float scale, void* workspace, size_t workspace_bytes,
                                    bool clear_counters, hipStream_t stream) {
  using namespace sgmv;
  if (num_slices < 1 || num_slices > SGMV_MAX_SLICES)
    return fail(SGMV_ERR_INVALID_ARGUMENT, "num_slices must be in 1..%d, got %d",
                SGMV_MAX_SLICES, num_slices);
  if (!known_dtype(x.dtype)) return fail(SGMV_ERR_INVALID_ARGUMENT, "unknown inputs dtype %d", x.dtype);
  if (x.rows < 0 || x.cols < 1 || x.row_stride < x.cols)
    return fail(SGMV_ERR_INVALID_ARGUMENT,
                "inputs shape (%lld, %lld) with row stride %lld is invalid", (long long)x.rows,
                (long long)x.cols, (long long)x.row_stride);
  if (x.rows > INT32_MAX)
    return fail(SGMV_ERR_UNSUPPORTED, "more than 2^31-1 tokens (%lld)", (long long)x.rows);
  if (x.cols > INT32_MAX) return fail(SGMV_ERR_UNSUPPORTED, "hidden size exceeds 2^31-1");
  if (batches < 0) return fail(SGMV_ERR_INVALID_ARGUMENT, "batches must be >= 0");
  if (batches > SGMV_MAX_BATCHES)
    return fail(SGMV_ERR_UNSUPPORTED, "batches %lld exceeds %d", (long long)batches,
                SGMV_MAX_BATCHES);
  if (max_seq_len < 0) return fail(SGMV_ERR_INVALID_ARGUMENT, "max_seq_len must be >= 0");
  const sgmv_shrink_slice& s0 = slices[0];
  const int64_t K = s0.lora_a.rows;
  const int64_t L = s0.lora_a.num;
  for (int i = 0; i < num_slices; ++i) {
    const sgmv_shrink_slice& s = slices[i];
    if (!known_dtype(s.lora_a.dtype) || !known_dtype(s.out.dtype))
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: unknown dtype", i);
    if (s.lora_a.dtype == SGMV_F32)
      return fail(SGMV_ERR_UNSUPPORTED, "slice %d: lora_a must be float16 or bfloat16", i);
    if (x.dtype != s.lora_a.dtype && x.dtype != SGMV_F32)
      return fail(SGMV_ERR_UNSUPPORTED,
                  "slice %d: inputs must have lora_a's dtype or float32 (got %d with %d)", i,
                  x.dtype, s.lora_a.dtype);
    if (s.lora_a.num < 0 || s.lora_a.rows < 1 || s.lora_a.cols < 1)
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: lora_a shape is invalid", i);
    if (s.lora_a.cols != x.cols)
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: lora_a hidden %lld != inputs hidden %lld",
                  i, (long long)s.lora_a.cols, (long long)x.cols);
    if (s.out.rows != x.rows || s.out.cols != s.lora_a.rows || s.out.row_stride < s.out.cols)
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: output (%lld, %lld) with row stride %lld must be (%lld, %lld)", i,
                  (long long)s.out.rows, (long long)s.out.cols, (long long)s.out.row_stride,
                  (long long)x.rows, (long long)s.lora_a.rows);
    if (i > 0 && (s.lora_a.rows != K || s.lora_a.num != L || s.lora_a.dtype != s0.lora_a.dtype ||
                  s.out.dtype != s0.out.dtype))
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "slice %d: rank, lora_num and dtypes must match slice 0", i);
  }
  if (K > SGMV_MAX_RANK)
    return fail(SGMV_ERR_UNSUPPORTED, "rank %lld exceeds %d", (long long)K, SGMV_MAX_RANK);
  if (L > INT32_MAX) return fail(SGMV_ERR_UNSUPPORTED, "lora_num exceeds 2^31-1");
  if (batches == 0 || x.rows == 0) {
    g_error.clear();
    return SGMV_OK;  // nothing to do
  }
  if (!x.data) return fail(SGMV_ERR_INVALID_ARGUMENT, "inputs data pointer is null");
  if (!start || !lens || !idx)
    return fail(SGMV_ERR_INVALID_ARGUMENT, "segment metadata pointer is null");
  for (int i = 0; i < num_slices; ++i)
    if (!slices[i].out.data || (!slices[i].lora_a.data && L > 0))
      return fail(SGMV_ERR_INVALID_ARGUMENT, "slice %d: null data pointer", i);
  if (workspace) {
    int cus = 0;
    const hipError_t e = device_compute_units(&cus);
    if (e != hipSuccess)
      return fail(SGMV_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
    const int64_t need = sgmv::limits::shrink_workspace_bytes(cus);
    if (!aligned16(workspace) || (int64_t)workspace_bytes < need)
      return fail(SGMV_ERR_INVALID_ARGUMENT,
                  "workspace must be 16-byte aligned and hold %lld bytes (got %zu)",
                  (long long)need, workspace_bytes);
  }

  // Fast kernels: 16-byte blocks everywhere, hidden < 2^26, a unit's rows
  // (64) of inputs or outputs spanning less than 2 GiB, and the lora_A rows
  // the k tiles address (16 k16 rows of one adapter's (K, H) block, the
  // rows past K masked) spanning less than 2 GiB as well: their buffer
  // offsets are 32-bit and the masked-lane offset 2^31 must lie past every
  // resource.  Decided for the inputs, then per slice; slices are launched
  // in runs that take the same kernel family (so a slice's result does not
  // depend on the others in the call).
  const int64_t xb = elem_bytes(x.dtype), ob = elem_bytes(s0.out.dtype);
  const int64_t span = kShrinkTokensSplitT;
  const int k16 = next_pow2((int)((K + 15) / 16));
  const bool fast_x = K % 8 == 0 && x.cols % 8 == 0 && x.cols < (int64_t(1) << 26) &&
                      shrink_fast_lora_a_fits(K, x.cols) &&
                      aligned16(x.data) && (x.row_stride * xb) % 16 == 0 &&
                      span * x.row_stride * xb < (int64_t(1) << 31);
  auto fast_slice = [&](int i) {
    const sgmv_shrink_slice& s = slices[i];
    return fast_x && aligned16(s.lora_a.data) && aligned16(s.out.data) &&
           (s.out.row_stride * ob) % 16 == 0 && span * s.out.row_stride * ob < (int64_t(1) << 31);
  };
  // The fast kernels take up to kShrinkMaxSlicesPerLaunch slices and 16 k
  // tiles of 16 rows per launch: more slices go in several launches (each
  // reads the inputs again).
  int fast_per_launch = 16 / k16;
  if (fast_per_launch > kShrinkMaxSlicesPerLaunch) fast_per_launch = kShrinkMaxSlicesPerLaunch;
  const int64_t units64 = (x.rows + kShrinkTokensSplitT - 1) / kShrinkTokensSplitT;
  const bool split_t = units64 >= shrink_split_t_min_units(k16) ||
                       (workspace && k16 >= 8 && units64 >= SGMV_SHRINK_SPLIT_T_MIN_UNITS_WIDE);
  if (clear_counters && workspace) {
    const sgmv_status st = clear_workspace_counters(workspace, stream);
    if (st != SGMV_OK) return st;
  }
  for (int first = 0; first < num_slices;) {
    const bool fast = fast_slice(first);
    const int limit = fast ? fast_per_launch : num_slices;
    int count = 1;
    while (first + count < num_slices && count < limit && fast_slice(first + count) == fast)
      ++count;
    const sgmv_status st = shrink_launch(x, slices, first, count, start, lens, idx, batches,
                                         scale, fast, split_t, workspace, stream);
    if (st != SGMV_OK) return st;
    first += count;
  }
  g_error.clear();
  return SGMV_OK;
}

}  // namespace

extern "C" {

sgmv_status sgmv_shrink(sgmv_matrix inputs, sgmv_stack lora_a, sgmv_matrix out,
                        const int64_t* b_seq_start_loc, const int64_t* seq_lens,
                        const int64_t* lora_indices, int64_t batches, int64_t max_seq_len,
                        float scale, void* workspace, size_t workspace_bytes,
                        hipStream_t stream) {
  sgmv_shrink_slice s;
  s.lora_a = lora_a;
  s.out = out;
  return shrink_check_and_launch(inputs, &s, 1, b_seq_start_loc, seq_lens, lora_indices, batches,
                                 max_seq_len, scale, workspace, workspace_bytes, false, stream);
}

sgmv_status sgmv_shrink_multi_slice(sgmv_matrix inputs, const sgmv_shrink_slice* slices,
                                    int num_slices, const int64_t* b_seq_start_loc,
                                    const int64_t* seq_lens, const int64_t* lora_indices,
                                    int64_t batches, int64_t max_seq_len, float scale,
                                    void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  if (!slices) return fail(SGMV_ERR_INVALID_ARGUMENT, "slices pointer is null");
  return shrink_check_and_launch(inputs, slices, num_slices, b_seq_start_loc, seq_lens,
                                 lora_indices, batches, max_seq_len, scale, workspace,
                                 workspace_bytes, false, stream);
}

sgmv_status sgmv_shrink_multi_slice_noalloc(sgmv_matrix inputs, const sgmv_shrink_slice* slices,
                                            int num_slices, const int64_t* b_seq_start_loc,
                                            const int64_t* seq_lens,
                                            const int64_t* lora_indices, int64_t batches,
                                            int64_t max_seq_len, float scale,
                                            hipStream_t stream) {
  if (!slices) return fail(SGMV_ERR_INVALID_ARGUMENT, "slices pointer is null");
  int cus = 0;
  hipError_t e = device_compute_units(&cus);
  if (e != hipSuccess) return fail(SGMV_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  const int64_t need = sgmv::limits::shrink_workspace_bytes(cus);
  if (need > kNoAllocBytes)
    return fail(SGMV_ERR_UNSUPPORTED,
                "the static workspace covers %d compute units (%lld bytes); this device has %d "
                "(use sgmv_shrink_multi_slice with a workspace)",
                kNoAllocMaxCus, (long long)kNoAllocBytes, cus);
  void* ws = nullptr;
  e = noalloc_workspace(&ws);
  if (e != hipSuccess)
    return fail(SGMV_ERR_HIP, "static workspace lookup failed: %s", hipGetErrorString(e));
  return shrink_check_and_launch(inputs, slices, num_slices, b_seq_start_loc, seq_lens,
                                 lora_indices, batches, max_seq_len, scale, ws, (size_t)need,
                                 true, stream);
}

sgmv_status sgmv_shrink_workspace_bytes(size_t* bytes) {
  if (!bytes) return fail(SGMV_ERR_INVALID_ARGUMENT, "bytes pointer is null");
  int cus = 0;
  const hipError_t e = device_compute_units(&cus);
  if (e != hipSuccess) return fail(SGMV_ERR_HIP, "device query failed: %s", hipGetErrorString(e));
  *bytes = (size_t)sgmv::limits::shrink_workspace_bytes(cus);
  g_error.clear();
  return SGMV_OK;
}

}  // extern "C"

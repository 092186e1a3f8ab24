// sgmv_stream.hip -- streaming-bandwidth probes for the benchmark (built into
// libsgmv_stream.so, separate from libsgmv): a kernel that reads R and
// writes W 16-byte vectors of HBM with the access forms the SGMV kernels
// use (16-byte buffer loads, non-temporal loads of streamed data, and
// non-temporal device-scope stores), so that a workload's achieved rate can
// be set against what plain streaming of the same traffic mix reaches on
// the same device.  Not part of the SGMV operation.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kLoadNT = 0x2;    // nt
constexpr int kStoreNT = 0x12;  // nt | sc1

// Grid-stride walk over max(R, W) positions, UNROLL positions per thread and
// iteration (independent accesses in flight).  With R <= W, position i
// writes vector i and, when (i R mod W) < R, also reads vector floor(i R /
// W): every read vector exactly once, the reads spread evenly among the
// writes (and the other way round for R > W).  The quotient and remainder
// advance incrementally along a thread's positions (one division per
// thread).  The XOR of what was read goes to sink only if it equals a value
// the data never produce, so the loads cannot be dropped and nothing else is
// written.
template <int UNROLL>
__global__ __launch_bounds__(kThreads) void stream_mix(const u32x4* __restrict__ src, uint64_t R,
                                                       u32x4* __restrict__ dst, uint64_t W,
                                                       uint32_t* __restrict__ sink,
                                                       uint32_t fill) {
  const uint64_t n = R > W ? R : W;
  const uint64_t lo = R > W ? W : R;  // the sparser stream
  const bool reads_dense = R > W;
  const uint64_t stride = (uint64_t)gridDim.x * kThreads;
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<u32x4*>(src), (short)0, 0x7fffffff, 0x00020000);
  __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc(dst, (short)0, 0x7fffffff, 0x00020000);
  const u32x4 v = {fill, fill ^ 1u, fill ^ 2u, fill ^ 3u};
  uint32_t acc = 0;
  const uint64_t i0 = (uint64_t)blockIdx.x * kThreads + threadIdx.x;
  if (n == 0 || i0 >= n) return;
  // position i0 + u stride of this thread: sparse index j[u], remainder rem[u]
  uint64_t j[UNROLL], rem[UNROLL];
#pragma unroll
  for (int u = 0; u < UNROLL; ++u) {
    const uint64_t i = i0 + (uint64_t)u * stride;
    j[u] = i * lo / n;
    rem[u] = i * lo % n;
  }
  const uint64_t step = stride * UNROLL;
  const uint64_t dq = step * lo / n, dr = step * lo % n;
  for (uint64_t i = i0; i < n; i += step) {
    u32x4 x[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint64_t iu = i + (uint64_t)u * stride;
      const bool in = iu < n;
      const bool sparse = rem[u] < lo;
      const uint64_t r_idx = reads_dense ? iu : j[u];
      x[u] = u32x4{0u, 0u, 0u, 0u};
      if (in && (reads_dense ? true : sparse) && R > 0)
        x[u] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(r_idx * 16), 0, kLoadNT));
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint64_t iu = i + (uint64_t)u * stride;
      const bool in = iu < n;
      const bool sparse = rem[u] < lo;
      const uint64_t w_idx = reads_dense ? j[u] : iu;
      if (in && (reads_dense ? sparse : true) && W > 0)
        __builtin_amdgcn_raw_buffer_store_b128(v, rd, (int)(w_idx * 16), 0, kStoreNT);
      acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
      j[u] += dq;
      rem[u] += dr;
      if (rem[u] >= n) {
        rem[u] -= n;
        ++j[u];
      }
    }
  }
  if (acc == 0x9e3779b9u && fill == 0x7f4a7c15u) sink[blockIdx.x & 255] = acc;
}

}  // namespace

extern "C" {

// Enqueue one probe on `stream`: read `read_bytes` from `src` and write
// `write_bytes` to `dst` (device buffers of at least those sizes, both
// multiples of 16 and below 2 GiB; 16-byte aligned), with `blocks`
// workgroups of 256 threads, each thread keeping `unroll` (1 or 4)
// accesses in flight; `sink`: 256 device words, written only in a case that
// does not occur.  Returns a hipError_t code.
int sgmv_stream_probe(const void* src, uint64_t read_bytes, void* dst, uint64_t write_bytes,
                      uint32_t* sink, int blocks, int unroll, hipStream_t stream) {
  if (read_bytes % 16 || write_bytes % 16 || read_bytes >= (1ull << 31) ||
      write_bytes >= (1ull << 31) || blocks < 1 || (unroll != 1 && unroll != 4))
    return (int)hipErrorInvalidValue;
  if ((read_bytes && !src) || (write_bytes && !dst) || !sink) return (int)hipErrorInvalidValue;
  if (unroll == 4)
    hipLaunchKernelGGL(stream_mix<4>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), read_bytes / 16, static_cast<u32x4*>(dst),
                       write_bytes / 16, sink, 0x5a5a5a5au);
  else
    hipLaunchKernelGGL(stream_mix<1>, dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(src), read_bytes / 16, static_cast<u32x4*>(dst),
                       write_bytes / 16, sink, 0x5a5a5a5au);
  return (int)hipGetLastError();
}

}  // extern "C"

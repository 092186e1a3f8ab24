// sgmv_c_client -- a plain C-ABI client of libsgmv: no Python and no torch,
// only the HIP runtime and include/sgmv.h.  It reads one problem from raw
// files, copies it to the GPU, enqueues the call on a stream of its own,
// copies the result back and writes it out.  It does no arithmetic of its
// own: the GPU tests prepare the files from a seeded workload and check the
// result with the oracle.
//
// usage: sgmv_c_client <mode> <dir>, mode one of
//   expand  sgmv_expand_slice.  problem.txt: "T K N H L offset xd wd od add
//           batches"; x.bin (T x K, xd), w.bin (L x N x K, wd)
//   multi   sgmv_expand_multi_slice.  problem.txt: "T K H L S xd wd od add
//           batches", then S lines "N offset"; x<i>.bin (T x K, xd) and
//           w<i>.bin (L x N_i x K, wd) per slice i
//   shrink  sgmv_shrink with a workspace of sgmv_shrink_workspace_bytes().
//           problem.txt: "T H K L xd wd od scale batches"; x.bin (T x H,
//           xd), a.bin (L x K x H, wd)
//   fused   sgmv_fused_shrink_expand.  problem.txt: "T H K L S xd wd od add
//           batches scale H_out", then S lines "N offset"; x.bin (T x H,
//           xd), a<i>.bin (L x K x H, wd), b<i>.bin (L x N_i x K, wd)
// and, for every mode, out0.bin (the prior output: T x H for expand and
// multi, T x K for shrink, T x H_out for fused, od) and start.bin,
// lens.bin, idx.bin (int64[batches]); the result goes to out.bin in
// out0.bin's layout.  Dtype codes are sgmv_dtype's (0 f16, 1 bf16, 2 f32).
// Exit status 0 on success; 1 with a message on stderr for any failure (bad
// arguments or files, a HIP error, a library status other than SGMV_OK).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "sgmv.h"

namespace {

int64_t elem_size(int dtype) { return dtype == SGMV_F32 ? 4 : 2; }
bool known(int dtype) { return dtype == SGMV_F16 || dtype == SGMV_BF16 || dtype == SGMV_F32; }

bool read_file(const std::string& path, std::vector<char>* data, int64_t expect_bytes) {
  FILE* f = fopen(path.c_str(), "rb");
  if (!f) {
    fprintf(stderr, "sgmv_c_client: cannot open %s\n", path.c_str());
    return false;
  }
  data->assign((size_t)expect_bytes, 0);
  const size_t got = expect_bytes > 0 ? fread(data->data(), 1, (size_t)expect_bytes, f) : 0;
  const bool extra = fgetc(f) != EOF;
  fclose(f);
  if ((int64_t)got != expect_bytes || extra) {
    fprintf(stderr, "sgmv_c_client: %s does not hold %lld bytes\n", path.c_str(),
            (long long)expect_bytes);
    return false;
  }
  return true;
}

bool write_file(const std::string& path, const std::vector<char>& data) {
  FILE* f = fopen(path.c_str(), "wb");
  if (!f) {
    fprintf(stderr, "sgmv_c_client: cannot create %s\n", path.c_str());
    return false;
  }
  const size_t put = data.empty() ? 0 : fwrite(data.data(), 1, data.size(), f);
  const bool ok = put == data.size() && fclose(f) == 0;
  if (!ok) fprintf(stderr, "sgmv_c_client: cannot write %s\n", path.c_str());
  return ok;
}

bool hip_ok(hipError_t e, const char* what) {
  if (e == hipSuccess) return true;
  fprintf(stderr, "sgmv_c_client: %s: %s\n", what, hipGetErrorString(e));
  return false;
}

bool library_ok(sgmv_status st, const char* call) {
  if (st == SGMV_OK) return true;
  fprintf(stderr, "sgmv_c_client: %s returned %d: %s\n", call, (int)st, sgmv_last_error());
  return false;
}

// Device copies of host buffers and a stream, released on destruction.
struct Device {
  std::vector<void*> ptrs;
  hipStream_t stream = nullptr;
  ~Device() {
    if (stream) (void)hipStreamDestroy(stream);
    for (void* p : ptrs) (void)hipFree(p);
  }
  void* upload(const std::vector<char>& host) {
    void* p = nullptr;
    if (!hip_ok(hipMalloc(&p, host.size() ? host.size() : 1), "hipMalloc")) return nullptr;
    ptrs.push_back(p);
    if (!host.empty() && !hip_ok(hipMemcpy(p, host.data(), host.size(), hipMemcpyHostToDevice),
                                 "hipMemcpy to device"))
      return nullptr;
    return p;
  }
  // A zero-filled device buffer of `bytes`.
  void* zeros(size_t bytes) {
    void* p = nullptr;
    if (!hip_ok(hipMalloc(&p, bytes ? bytes : 1), "hipMalloc")) return nullptr;
    ptrs.push_back(p);
    if (!hip_ok(hipMemset(p, 0, bytes), "hipMemset") ||
        !hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize"))
      return nullptr;
    return p;
  }
};

// The segment metadata of a problem, on the host and the device.
struct Segments {
  std::vector<char> start, lens, idx;
  const int64_t *d_start = nullptr, *d_lens = nullptr, *d_idx = nullptr;
  int64_t max_len = 0;
  bool load(const std::string& dir, int64_t batches, Device* dev) {
    if (!read_file(dir + "/start.bin", &start, batches * 8) ||
        !read_file(dir + "/lens.bin", &lens, batches * 8) ||
        !read_file(dir + "/idx.bin", &idx, batches * 8))
      return false;
    for (int64_t b = 0; b < batches; ++b) {
      int64_t v;
      memcpy(&v, lens.data() + 8 * b, 8);
      if (v > max_len) max_len = v;
    }
    d_start = static_cast<const int64_t*>(dev->upload(start));
    d_lens = static_cast<const int64_t*>(dev->upload(lens));
    d_idx = static_cast<const int64_t*>(dev->upload(idx));
    return d_start && d_lens && d_idx;
  }
};

FILE* open_problem(const std::string& dir) {
  FILE* f = fopen((dir + "/problem.txt").c_str(), "r");
  if (!f) fprintf(stderr, "sgmv_c_client: cannot open %s/problem.txt\n", dir.c_str());
  return f;
}

bool bad_problem(const char* mode) {
  fprintf(stderr, "sgmv_c_client: bad %s problem.txt\n", mode);
  return false;
}

// Reads `count` "N offset" lines into widths / offsets.
bool read_windows(FILE* f, int count, std::vector<int64_t>* widths,
                  std::vector<int64_t>* offsets) {
  for (int i = 0; i < count; ++i) {
    long long n, off;
    if (fscanf(f, "%lld %lld", &n, &off) != 2 || n < 0 || off < 0) return false;
    widths->push_back(n);
    offsets->push_back(off);
  }
  return true;
}

// Waits for the stream, copies the output back and writes out.bin.
bool finish(Device* dev, void* d_out, std::vector<char>* out, const std::string& dir) {
  return hip_ok(hipStreamSynchronize(dev->stream), "hipStreamSynchronize") &&
         hip_ok(hipMemcpy(out->data(), d_out, out->size(), hipMemcpyDeviceToHost),
                "hipMemcpy to host") &&
         write_file(dir + "/out.bin", *out);
}

bool run_expand(const std::string& dir) {
  long long T, K, N, H, L, off, add, batches;
  int xd, wd, od;
  FILE* f = open_problem(dir);
  if (!f) return false;
  const int n = fscanf(f, "%lld %lld %lld %lld %lld %lld %d %d %d %lld %lld", &T, &K, &N, &H, &L,
                       &off, &xd, &wd, &od, &add, &batches);
  fclose(f);
  if (n != 11 || T < 0 || K < 1 || N < 0 || H < 1 || L < 1 || off < 0 || batches < 0 ||
      !known(xd) || !known(wd) || !known(od))
    return bad_problem("expand");
  std::vector<char> x, w, out;
  if (!read_file(dir + "/x.bin", &x, T * K * elem_size(xd)) ||
      !read_file(dir + "/w.bin", &w, L * N * K * elem_size(wd)) ||
      !read_file(dir + "/out0.bin", &out, T * H * elem_size(od)))
    return false;
  Device dev;
  Segments seg;
  if (!seg.load(dir, batches, &dev)) return false;
  void* dx = dev.upload(x);
  void* dw = dev.upload(w);
  void* dout = dev.upload(out);
  if (!dx || !dw || !dout || !hip_ok(hipStreamCreate(&dev.stream), "hipStreamCreate"))
    return false;
  const sgmv_matrix mx = {dx, xd, T, K, K};
  const sgmv_stack mw = {dw, wd, L, N, K};
  const sgmv_matrix mo = {dout, od, T, H, H};
  return library_ok(sgmv_expand_slice(mx, mw, mo, seg.d_start, seg.d_lens, seg.d_idx, batches,
                                      seg.max_len, off, N, (int)add, dev.stream),
                    "sgmv_expand_slice") &&
         finish(&dev, dout, &out, dir);
}

bool run_multi(const std::string& dir) {
  long long T, K, H, L, add, batches;
  int S, xd, wd, od;
  FILE* f = open_problem(dir);
  if (!f) return false;
  std::vector<int64_t> widths, offsets;
  const int n = fscanf(f, "%lld %lld %lld %lld %d %d %d %d %lld %lld", &T, &K, &H, &L, &S, &xd,
                       &wd, &od, &add, &batches);
  const bool windows = n == 10 && S >= 1 && S <= SGMV_MAX_SLICES &&
                       read_windows(f, S, &widths, &offsets);
  fclose(f);
  if (!windows || T < 0 || K < 1 || H < 1 || L < 1 || batches < 0 || !known(xd) ||
      !known(wd) || !known(od))
    return bad_problem("multi");
  Device dev;
  Segments seg;
  if (!seg.load(dir, batches, &dev)) return false;
  std::vector<sgmv_slice> slices(S);
  for (int i = 0; i < S; ++i) {
    std::vector<char> x, w;
    if (!read_file(dir + "/x" + std::to_string(i) + ".bin", &x, T * K * elem_size(xd)) ||
        !read_file(dir + "/w" + std::to_string(i) + ".bin", &w,
                   L * widths[i] * K * elem_size(wd)))
      return false;
    void* dx = dev.upload(x);
    void* dw = dev.upload(w);
    if (!dx || !dw) return false;
    slices[i].inputs = {dx, xd, T, K, K};
    slices[i].lora_b = {dw, wd, L, widths[i], K};
    slices[i].slice_offset = offsets[i];
    slices[i].slice_size = widths[i];
  }
  std::vector<char> out;
  if (!read_file(dir + "/out0.bin", &out, T * H * elem_size(od))) return false;
  void* dout = dev.upload(out);
  if (!dout || !hip_ok(hipStreamCreate(&dev.stream), "hipStreamCreate")) return false;
  const sgmv_matrix mo = {dout, od, T, H, H};
  return library_ok(sgmv_expand_multi_slice(slices.data(), S, mo, seg.d_start, seg.d_lens,
                                            seg.d_idx, batches, seg.max_len, (int)add,
                                            dev.stream),
                    "sgmv_expand_multi_slice") &&
         finish(&dev, dout, &out, dir);
}

bool run_shrink(const std::string& dir) {
  long long T, H, K, L, batches;
  int xd, wd, od;
  float scale;
  FILE* f = open_problem(dir);
  if (!f) return false;
  const int n = fscanf(f, "%lld %lld %lld %lld %d %d %d %f %lld", &T, &H, &K, &L, &xd, &wd, &od,
                       &scale, &batches);
  fclose(f);
  if (n != 9 || T < 0 || H < 1 || K < 1 || L < 1 || batches < 0 || !known(xd) || !known(wd) ||
      !known(od))
    return bad_problem("shrink");
  std::vector<char> x, a, out;
  if (!read_file(dir + "/x.bin", &x, T * H * elem_size(xd)) ||
      !read_file(dir + "/a.bin", &a, L * K * H * elem_size(wd)) ||
      !read_file(dir + "/out0.bin", &out, T * K * elem_size(od)))
    return false;
  Device dev;
  Segments seg;
  if (!seg.load(dir, batches, &dev)) return false;
  void* dx = dev.upload(x);
  void* da = dev.upload(a);
  void* dout = dev.upload(out);
  if (!dx || !da || !dout || !hip_ok(hipStreamCreate(&dev.stream), "hipStreamCreate"))
    return false;
  size_t ws_bytes = 0;
  if (!library_ok(sgmv_shrink_workspace_bytes(&ws_bytes), "sgmv_shrink_workspace_bytes"))
    return false;
  void* ws = dev.zeros(ws_bytes);
  if (!ws) return false;
  const sgmv_matrix mx = {dx, xd, T, H, H};
  const sgmv_stack ma = {da, wd, L, K, H};
  const sgmv_matrix mo = {dout, od, T, K, K};
  return library_ok(sgmv_shrink(mx, ma, mo, seg.d_start, seg.d_lens, seg.d_idx, batches,
                                seg.max_len, scale, ws, ws_bytes, dev.stream),
                    "sgmv_shrink") &&
         finish(&dev, dout, &out, dir);
}

bool run_fused(const std::string& dir) {
  long long T, H, K, L, add, batches, H_out;
  int S, xd, wd, od;
  float scale;
  FILE* f = open_problem(dir);
  if (!f) return false;
  std::vector<int64_t> widths, offsets;
  const int n = fscanf(f, "%lld %lld %lld %lld %d %d %d %d %lld %lld %f %lld", &T, &H, &K, &L, &S,
                       &xd, &wd, &od, &add, &batches, &scale, &H_out);
  const bool windows = n == 12 && S >= 1 && S <= SGMV_MAX_FUSED_SLICES &&
                       read_windows(f, S, &widths, &offsets);
  fclose(f);
  if (!windows || T < 0 || H < 1 || K < 1 || L < 1 || batches < 0 || H_out < 1 || !known(xd) ||
      !known(wd) || !known(od))
    return bad_problem("fused");
  Device dev;
  Segments seg;
  if (!seg.load(dir, batches, &dev)) return false;
  std::vector<char> x;
  if (!read_file(dir + "/x.bin", &x, T * H * elem_size(xd))) return false;
  void* dx = dev.upload(x);
  if (!dx) return false;
  std::vector<sgmv_fused_slice> slices(S);
  for (int i = 0; i < S; ++i) {
    std::vector<char> a, b;
    if (!read_file(dir + "/a" + std::to_string(i) + ".bin", &a, L * K * H * elem_size(wd)) ||
        !read_file(dir + "/b" + std::to_string(i) + ".bin", &b,
                   L * widths[i] * K * elem_size(wd)))
      return false;
    void* da = dev.upload(a);
    void* db = dev.upload(b);
    if (!da || !db) return false;
    slices[i].lora_a = {da, wd, L, K, H};
    slices[i].lora_b = {db, wd, L, widths[i], K};
    slices[i].slice_offset = offsets[i];
  }
  std::vector<char> out;
  if (!read_file(dir + "/out0.bin", &out, T * H_out * elem_size(od))) return false;
  void* dout = dev.upload(out);
  if (!dout || !hip_ok(hipStreamCreate(&dev.stream), "hipStreamCreate")) return false;
  const sgmv_matrix mx = {dx, xd, T, H, H};
  const sgmv_matrix mo = {dout, od, T, H_out, H_out};
  return library_ok(sgmv_fused_shrink_expand(mx, slices.data(), S, mo, seg.d_start, seg.d_lens,
                                             seg.d_idx, batches, seg.max_len, scale, (int)add,
                                             dev.stream),
                    "sgmv_fused_shrink_expand") &&
         finish(&dev, dout, &out, dir);
}

}  // namespace

int main(int argc, char** argv) {
  const char* modes[] = {"expand", "multi", "shrink", "fused"};
  int mode = -1;
  for (int i = 0; i < 4 && argc == 3; ++i)
    if (strcmp(argv[1], modes[i]) == 0) mode = i;
  if (mode < 0) {
    fprintf(stderr, "usage: sgmv_c_client expand|multi|shrink|fused <dir>\n");
    return 1;
  }
  if (sgmv_abi_version() != SGMV_ABI_VERSION) {
    fprintf(stderr, "sgmv_c_client: libsgmv ABI %d, header %d\n", sgmv_abi_version(),
            SGMV_ABI_VERSION);
    return 1;
  }
  const std::string dir = argv[2];
  const bool ok = mode == 0   ? run_expand(dir)
                  : mode == 1 ? run_multi(dir)
                  : mode == 2 ? run_shrink(dir)
                              : run_fused(dir);
  return ok ? 0 : 1;
}

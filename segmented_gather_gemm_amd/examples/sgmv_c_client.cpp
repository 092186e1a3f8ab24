// sgmv_c_client -- a plain C-ABI client of libsgmv: no Python and no torch,
// only the HIP runtime and include/sgmv.h.  It reads one problem from raw
// files, copies it to the GPU, enqueues the call on a stream of its own,
// copies the result back and writes it out.  It does no arithmetic of its
// own: the GPU tests prepare the files from a seeded workload and check the
// result with the oracle.
//
// usage: sgmv_c_client expand <dir>
//   <dir>/problem.txt  "T K N H L offset x_dtype w_dtype out_dtype add batches"
//   <dir>/x.bin (T x K, x_dtype), w.bin (L x N x K, w_dtype), out0.bin (T x H,
//   out_dtype), start.bin, lens.bin, idx.bin (int64[batches])
//   -> <dir>/out.bin (T x H, out_dtype), from sgmv_expand_slice
// usage: sgmv_c_client shrink <dir>
//   <dir>/problem.txt  "T H K L x_dtype a_dtype out_dtype scale batches"
//   <dir>/x.bin (T x H), a.bin (L x K x H), out0.bin (T x K), start.bin,
//   lens.bin, idx.bin
//   -> <dir>/out.bin (T x K), from sgmv_shrink
// Dtype codes are sgmv_dtype's (0 f16, 1 bf16, 2 f32).  Exit status 0 on
// success; 1 with a message on stderr for any failure (bad arguments or
// files, a HIP error, a library status other than SGMV_OK).
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

// Device copies of host buffers, freed on destruction.
struct DeviceBuffers {
  std::vector<void*> ptrs;
  ~DeviceBuffers() {
    for (void* p : ptrs) (void)hipFree(p);
  }
  void* upload(const std::vector<char>& host) {
    void* p = nullptr;
    const size_t n = host.size() ? host.size() : 1;
    if (!hip_ok(hipMalloc(&p, n), "hipMalloc")) return nullptr;
    ptrs.push_back(p);
    if (!host.empty() && !hip_ok(hipMemcpy(p, host.data(), host.size(), hipMemcpyHostToDevice),
                                 "hipMemcpy to device"))
      return nullptr;
    return p;
  }
};

bool library_ok(sgmv_status st, const char* call) {
  if (st == SGMV_OK) return true;
  fprintf(stderr, "sgmv_c_client: %s returned %d: %s\n", call, (int)st, sgmv_last_error());
  return false;
}

int run_expand(const std::string& dir) {
  long long T, K, N, H, L, off, add, batches;
  int xd, wd, od;
  FILE* f = fopen((dir + "/problem.txt").c_str(), "r");
  if (!f) {
    fprintf(stderr, "sgmv_c_client: cannot open %s/problem.txt\n", dir.c_str());
    return 1;
  }
  const int n = fscanf(f, "%lld %lld %lld %lld %lld %lld %d %d %d %lld %lld", &T, &K, &N, &H, &L,
                       &off, &xd, &wd, &od, &add, &batches);
  fclose(f);
  if (n != 11 || T < 0 || K < 1 || N < 0 || H < 1 || L < 1 || off < 0 || batches < 0 ||
      !known(xd) || !known(wd) || !known(od)) {
    fprintf(stderr, "sgmv_c_client: bad expand problem.txt\n");
    return 1;
  }
  std::vector<char> x, w, out, start, lens, idx;
  if (!read_file(dir + "/x.bin", &x, T * K * elem_size(xd)) ||
      !read_file(dir + "/w.bin", &w, L * N * K * elem_size(wd)) ||
      !read_file(dir + "/out0.bin", &out, T * H * elem_size(od)) ||
      !read_file(dir + "/start.bin", &start, batches * 8) ||
      !read_file(dir + "/lens.bin", &lens, batches * 8) ||
      !read_file(dir + "/idx.bin", &idx, batches * 8))
    return 1;
  DeviceBuffers dev;
  void* dx = dev.upload(x);
  void* dw = dev.upload(w);
  void* dout = dev.upload(out);
  void* dstart = dev.upload(start);
  void* dlens = dev.upload(lens);
  void* didx = dev.upload(idx);
  if (!dx || !dw || !dout || !dstart || !dlens || !didx) return 1;
  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
  const sgmv_matrix mx = {dx, xd, T, K, K};
  const sgmv_stack mw = {dw, wd, L, N, K};
  const sgmv_matrix mo = {dout, od, T, H, H};
  int64_t max_len = 0;
  for (long long b = 0; b < batches; ++b) {
    int64_t v;
    memcpy(&v, lens.data() + 8 * b, 8);
    if (v > max_len) max_len = v;
  }
  const sgmv_status st = sgmv_expand_slice(
      mx, mw, mo, static_cast<const int64_t*>(dstart), static_cast<const int64_t*>(dlens),
      static_cast<const int64_t*>(didx), batches, max_len, off, N, (int)add, stream);
  bool ok = library_ok(st, "sgmv_expand_slice") &&
            hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize") &&
            hip_ok(hipMemcpy(out.data(), dout, out.size(), hipMemcpyDeviceToHost),
                   "hipMemcpy to host");
  (void)hipStreamDestroy(stream);
  return ok && write_file(dir + "/out.bin", out) ? 0 : 1;
}

int run_shrink(const std::string& dir) {
  long long T, H, K, L, batches;
  int xd, ad, od;
  float scale;
  FILE* f = fopen((dir + "/problem.txt").c_str(), "r");
  if (!f) {
    fprintf(stderr, "sgmv_c_client: cannot open %s/problem.txt\n", dir.c_str());
    return 1;
  }
  const int n = fscanf(f, "%lld %lld %lld %lld %d %d %d %f %lld", &T, &H, &K, &L, &xd, &ad, &od,
                       &scale, &batches);
  fclose(f);
  if (n != 9 || T < 0 || H < 1 || K < 1 || L < 1 || batches < 0 || !known(xd) || !known(ad) ||
      !known(od)) {
    fprintf(stderr, "sgmv_c_client: bad shrink problem.txt\n");
    return 1;
  }
  std::vector<char> x, a, out, start, lens, idx;
  if (!read_file(dir + "/x.bin", &x, T * H * elem_size(xd)) ||
      !read_file(dir + "/a.bin", &a, L * K * H * elem_size(ad)) ||
      !read_file(dir + "/out0.bin", &out, T * K * elem_size(od)) ||
      !read_file(dir + "/start.bin", &start, batches * 8) ||
      !read_file(dir + "/lens.bin", &lens, batches * 8) ||
      !read_file(dir + "/idx.bin", &idx, batches * 8))
    return 1;
  DeviceBuffers dev;
  void* dx = dev.upload(x);
  void* da = dev.upload(a);
  void* dout = dev.upload(out);
  void* dstart = dev.upload(start);
  void* dlens = dev.upload(lens);
  void* didx = dev.upload(idx);
  if (!dx || !da || !dout || !dstart || !dlens || !didx) return 1;
  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
  const sgmv_matrix mx = {dx, xd, T, H, H};
  const sgmv_stack ma = {da, ad, L, K, H};
  const sgmv_matrix mo = {dout, od, T, K, K};
  int64_t max_len = 0;
  for (long long b = 0; b < batches; ++b) {
    int64_t v;
    memcpy(&v, lens.data() + 8 * b, 8);
    if (v > max_len) max_len = v;
  }
  const sgmv_status st = sgmv_shrink(mx, ma, mo, static_cast<const int64_t*>(dstart),
                                     static_cast<const int64_t*>(dlens),
                                     static_cast<const int64_t*>(didx), batches, max_len, scale,
                                     stream);
  bool ok = library_ok(st, "sgmv_shrink") &&
            hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize") &&
            hip_ok(hipMemcpy(out.data(), dout, out.size(), hipMemcpyDeviceToHost),
                   "hipMemcpy to host");
  (void)hipStreamDestroy(stream);
  return ok && write_file(dir + "/out.bin", out) ? 0 : 1;
}

}  // namespace

int main(int argc, char** argv) {
  if (argc != 3 || (strcmp(argv[1], "expand") != 0 && strcmp(argv[1], "shrink") != 0)) {
    fprintf(stderr, "usage: sgmv_c_client expand|shrink <dir>\n");
    return 1;
  }
  if (sgmv_abi_version() != SGMV_ABI_VERSION) {
    fprintf(stderr, "sgmv_c_client: libsgmv ABI %d, header %d\n", sgmv_abi_version(),
            SGMV_ABI_VERSION);
    return 1;
  }
  return strcmp(argv[1], "expand") == 0 ? run_expand(argv[2]) : run_shrink(argv[2]);
}

// sgmv_host.cpp -- definitions of the host helpers shared by libsgmv's entry
// points (see sgmv_host.h): the per-thread error message and the cached
// device capacity query.
#include <cstdarg>
#include <cstdio>
#include <map>
#include <mutex>
#include <string>
#include <tuple>

#include "sgmv_host.h"
#include "sgmv_launch.h"

namespace sgmv {
namespace host {

thread_local std::string g_error;

sgmv_status fail(sgmv_status status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return status;
}

// Per-device compute-unit counts and per-(device, kernel, LDS bucket)
// occupancy, computed once.
std::mutex g_mu;
std::map<int, int> g_cus;
std::map<std::tuple<int, const void*, size_t>, int> g_occupancy;

// The entry for `dev` in g_cus, filled on first use (g_mu held).
static hipError_t cached_cus(int dev, std::map<int, int>::iterator* it) {
  auto cu = g_cus.find(dev);
  if (cu == g_cus.end()) {
    int n = 0;
    const hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cu = g_cus.emplace(dev, n > 0 ? n : 1).first;
  }
  *it = cu;
  return hipSuccess;
}

hipError_t device_compute_units(int* compute_units) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  std::map<int, int>::iterator cu;
  e = cached_cus(dev, &cu);
  if (e != hipSuccess) return e;
  *compute_units = cu->second;
  return hipSuccess;
}

hipError_t device_capacity(const void* kernel, size_t lds_bytes, int* workgroups,
                           int* compute_units) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const size_t bucket = (lds_bytes + 4095) / 4096 * 4096;
  std::lock_guard<std::mutex> lock(g_mu);
  std::map<int, int>::iterator cu;
  e = cached_cus(dev, &cu);
  if (e != hipSuccess) return e;
  const auto key = std::make_tuple(dev, kernel, bucket);
  auto occ = g_occupancy.find(key);
  if (occ == g_occupancy.end()) {
    int blocks = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, sgmv::kThreads, bucket);
    if (e != hipSuccess) return e;
    occ = g_occupancy.emplace(key, blocks > 0 ? blocks : 0).first;
  }
  *workgroups = cu->second * occ->second;
  if (compute_units) *compute_units = cu->second;
  return hipSuccess;
}

}  // namespace host
}  // namespace sgmv

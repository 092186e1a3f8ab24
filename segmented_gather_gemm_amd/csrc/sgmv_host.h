// sgmv_host.h -- host-side helpers shared by libsgmv's entry points
// (sgmv_api.cpp: the expand; sgmv_shrink_api.cpp: the LoRA-A projection).
// Internal to libsgmv.
#pragma once

#include <stdint.h>

#include <string>

#include "sgmv.h"

namespace sgmv {
namespace host {

// Message of the last non-OK status on this thread (sgmv_last_error).
extern thread_local std::string g_error;

// Record a printf-style message and return `status`.
sgmv_status fail(sgmv_status status, const char* fmt, ...);

inline bool known_dtype(int32_t d) { return d == SGMV_F16 || d == SGMV_BF16 || d == SGMV_F32; }
inline int64_t elem_bytes(int32_t d) { return d == SGMV_F32 ? 4 : 2; }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Workgroups of `kernel` (block of sgmv::kThreads threads, `lds_bytes` of
// dynamic LDS) that fit the current device at once: compute units times
// resident blocks per unit, queried once per (device, kernel, LDS bucket);
// 0 when one workgroup does not fit a compute unit.  The device's compute
// unit count goes to *compute_units when that is not null.
hipError_t device_capacity(const void* kernel, size_t lds_bytes, int* workgroups,
                           int* compute_units = nullptr);

// The current device's compute-unit count (cached per device, as above).
hipError_t device_compute_units(int* compute_units);

}  // namespace host
}  // namespace sgmv

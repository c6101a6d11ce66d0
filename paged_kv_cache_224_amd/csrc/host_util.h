// host_util.h -- small host-side helpers shared by the library's translation units
// (argument checks, the PKV_CHECK switch, launch status, synchronous device-to-host copies).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <vector>

#include "pagedkv.h"

namespace pkv_host {

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline bool check_mode() {
  const char* e = getenv("PKV_CHECK");
  return e && e[0] == '1' && e[1] == '\0';
}

inline int launch_status() {
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

template <typename T>
inline bool copy_to_host(std::vector<T>& dst, const T* src, size_t n, hipStream_t st) {
  dst.resize(n);
  if (n == 0) return true;
  if (hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDeviceToHost, st) != hipSuccess)
    return false;
  return hipStreamSynchronize(st) == hipSuccess;
}

}  // namespace pkv_host

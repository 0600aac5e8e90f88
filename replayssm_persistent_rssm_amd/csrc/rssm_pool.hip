// rssm_pool.hip -- physically contiguous device memory for state pools (the
// C ABI is declared in rssm_pool.h).
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <sys/types.h>

#include "rssm_pool.h"

namespace {

// Allocate on the current device: contiguous when the device has such a
// range, otherwise plain device memory.
void* pool_alloc(size_t bytes, int32_t* contiguous) {
  void* p = nullptr;
  if (hipExtMallocWithFlags(&p, bytes, hipDeviceMallocContiguous) == hipSuccess) {
    if (contiguous != nullptr) *contiguous = 1;
    return p;
  }
  (void)hipGetLastError();   // clear the failed attempt's error
  p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  if (contiguous != nullptr) *contiguous = 0;
  return p;
}

// Run f with `device` current, restoring the caller's device.
template <class F>
auto on_device(int device, F f) -> decltype(f()) {
  int cur = -1;
  const bool have = hipGetDevice(&cur) == hipSuccess;
  if (have && cur != device) (void)hipSetDevice(device);
  auto r = f();
  if (have && cur != device) (void)hipSetDevice(cur);
  return r;
}

}  // namespace

extern "C" {

rssm_status rssm_pool_alloc(uint64_t bytes, void** out, int32_t* contiguous) {
  if (out == nullptr) return RSSM_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (bytes == 0) return RSSM_ERR_INVALID_ARGUMENT;
  void* p = pool_alloc(static_cast<size_t>(bytes), contiguous);
  if (p == nullptr) return RSSM_ERR_HIP;
  *out = p;
  return RSSM_OK;
}

rssm_status rssm_pool_free(void* ptr) {
  if (ptr == nullptr) return RSSM_OK;
  // the device may still run work that reads the pool
  if (hipDeviceSynchronize() != hipSuccess || hipFree(ptr) != hipSuccess) {
    (void)hipGetLastError();
    return RSSM_ERR_HIP;
  }
  return RSSM_OK;
}

void* rssm_torch_pool_alloc(ssize_t bytes, int device, void* stream) {
  (void)stream;
  return on_device(device, [&] { return pool_alloc(bytes > 0 ? static_cast<size_t>(bytes) : 1, nullptr); });
}

void rssm_torch_pool_free(void* ptr, ssize_t bytes, int device, void* stream) {
  (void)bytes;
  (void)stream;
  on_device(device, [&] { return rssm_pool_free(ptr); });
}

}  // extern "C"

// Device memory for an arena laid out by zero_arena_layout. The layout's staggers rely on the
// arena's physical pages following its virtual addresses, which a physically contiguous
// allocation guarantees; an ordinary allocation usually, but not always, comes close. These two
// calls are the library's only allocations, made on request and never inside a step.
#include <hip/hip_runtime_api.h>

#include "zero_internal.h"

extern "C" {

zero_status zero_arena_alloc(uint64_t bytes, void** d_ptr, int32_t* contiguous) {
  const char* fn = "zero_arena_alloc";
  if (!d_ptr) return zero::fail(ZERO_E_INVAL, "%s: d_ptr is NULL", fn);
  *d_ptr = nullptr;
  if (contiguous) *contiguous = 0;
  if (bytes == 0) return zero::ok();
  void* p = nullptr;
  hipError_t e = hipExtMallocWithFlags(&p, bytes, hipDeviceMallocContiguous);
  if (e == hipSuccess) {
    *d_ptr = p;
    if (contiguous) *contiguous = 1;
    return zero::ok();
  }
  (void)hipGetLastError();  // the contiguous request failed: clear it and ask for ordinary memory
  e = hipMalloc(&p, bytes);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return zero::fail(ZERO_E_HIP, "%s: %llu bytes: %s", fn, (unsigned long long)bytes,
                      hipGetErrorString(e));
  }
  *d_ptr = p;
  return zero::ok();
}

zero_status zero_arena_free(void* d_ptr) {
  if (!d_ptr) return zero::ok();
  const hipError_t e = hipFree(d_ptr);
  if (e != hipSuccess) return zero::fail(ZERO_E_HIP, "zero_arena_free: %s", hipGetErrorString(e));
  return zero::ok();
}

}  // extern "C"

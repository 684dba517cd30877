// Device-side helpers shared by the kernels of libzero_shard: vector types and the streaming
// (non-temporal) loads and stores every kernel uses, since each byte is touched once per call.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#ifndef ZERO_NT
#define ZERO_NT 1  // non-temporal loads and stores
#endif

namespace zero {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ld(const T* p) {
#if ZERO_NT
  return __builtin_nontemporal_load(p);
#else
  return *p;
#endif
}

template <typename T>
__device__ __forceinline__ void st(T* p, T v) {
#if ZERO_NT
  __builtin_nontemporal_store(v, p);
#else
  *p = v;
#endif
}

}  // namespace zero

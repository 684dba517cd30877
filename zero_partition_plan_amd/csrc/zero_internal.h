// Internal helpers shared by the host-side translation units of libzero_shard.
#pragma once

#include <stdint.h>

#include "zero_shard.h"

namespace zero {

// Records a formatted message as this thread's last error and returns `s`.
zero_status fail(zero_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears this thread's last error and returns ZERO_OK.
zero_status ok();

// True when [a, a + abytes) and [b, b + bbytes) share a byte (empty ranges never overlap).
inline bool overlaps(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
  if (abytes == 0 || bbytes == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bbytes && y < x + abytes;
}

inline uint32_t dtype_bytes(int32_t dt) { return dt == ZERO_F32 ? 4u : 2u; }

inline bool dtype_valid(int32_t dt) { return dt == ZERO_F32 || dt == ZERO_F16 || dt == ZERO_BF16; }

}  // namespace zero

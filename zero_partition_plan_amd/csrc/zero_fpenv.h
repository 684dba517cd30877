// Host floating-point mode for the library's host arithmetic (x86-64 only; no device code includes
// this header).
#pragma once

#include <xmmintrin.h>

namespace zero {

// The SSE control register of the running thread set to IEEE behaviour (round to nearest, no
// flush-to-zero, no denormals-are-zero) for the scope, and restored after it. The host update and
// the fp64 derivation of the step constants run under it, so they give the bits the kernels and
// the oracle give whatever floating-point mode the caller's threads (and so the worker threads,
// which start with a copy of it) run in.
class IeeeScope {
 public:
  IeeeScope() : saved_(_mm_getcsr()) { _mm_setcsr(saved_ & ~kNonIeee); }
  ~IeeeScope() { _mm_setcsr(saved_); }
  IeeeScope(const IeeeScope&) = delete;
  IeeeScope& operator=(const IeeeScope&) = delete;

 private:
  static constexpr unsigned kNonIeee = 0x8000u | 0x6000u | 0x0040u;  // FTZ, rounding control, DAZ
  unsigned saved_;
};

}  // namespace zero

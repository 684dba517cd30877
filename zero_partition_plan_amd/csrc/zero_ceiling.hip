// Measurement kernels for the benchmark's context legs; not part of the optimizer step. They move
// the bytes of a known access pattern with trivial arithmetic, on the step's own arrays, so that a
// benchmark line can state what this GPU's memory system gives that pattern in the same placement:
//   zero_ceiling_twin   the fused step's traffic: R 16-bit replica rows and master, m, v read;
//                       master, m, v and a 16-bit slot written; the same tile, lane mapping and
//                       non-temporal accesses as the update kernel, with x + c*acc for the math.
//   zero_ceiling_triad  a[i] = a[i] + s*b[i]: two fp32 read streams and one write stream.
// With c = 0 and s = 0 every array keeps its values (for finite data), so the legs can run on live
// state. Built as its own library (libzero_ceiling.so), loaded only by the benchmark.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zero_device.h"

namespace {

using zero::f32x4;
using zero::ld;
using zero::st;
using zero::u32x2;

constexpr int kReps = 8;                        // the 7B step's replica count
constexpr uint64_t kTile = 256;                 // 64 lanes x 4 elements
constexpr uint64_t kMaxGrid = 1u << 24;

struct Rows {
  const uint16_t* p[kReps];
};

__global__ __launch_bounds__(64) void k_twin(Rows reps, uint64_t first_tile, float* __restrict__ P,
                                             float* __restrict__ M, float* __restrict__ V,
                                             uint16_t* __restrict__ out, float c) {
  const uint64_t i = (first_tile + blockIdx.x) * kTile + threadIdx.x * 4u;
  f32x4 p = ld(reinterpret_cast<const f32x4*>(P + i));
  f32x4 m = ld(reinterpret_cast<const f32x4*>(M + i));
  f32x4 v = ld(reinterpret_cast<const f32x4*>(V + i));
  u32x2 w[kReps];
#pragma unroll
  for (int k = 0; k < kReps; ++k) w[k] = ld(reinterpret_cast<const u32x2*>(reps.p[k] + i));
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kReps; ++k) {
    acc.x += __uint_as_float(w[k].x << 16);
    acc.y += __uint_as_float(w[k].x & 0xffff0000u);
    acc.z += __uint_as_float(w[k].y << 16);
    acc.w += __uint_as_float(w[k].y & 0xffff0000u);
  }
  p = p + c * acc;
  m = m + c * acc;
  v = v + c * acc;
  st(reinterpret_cast<f32x4*>(P + i), p);
  st(reinterpret_cast<f32x4*>(M + i), m);
  st(reinterpret_cast<f32x4*>(V + i), v);
  // bf16 by truncation: the pattern's bytes, not the step's rounding, are what is measured here
  const u32x2 o = {(__float_as_uint(p.x) >> 16) | (__float_as_uint(p.y) & 0xffff0000u),
                   (__float_as_uint(p.z) >> 16) | (__float_as_uint(p.w) & 0xffff0000u)};
  st(reinterpret_cast<u32x2*>(out + i), o);
}

__global__ __launch_bounds__(64) void k_triad(float* __restrict__ a, const float* __restrict__ b,
                                              uint64_t first_tile, float s) {
  const uint64_t i = (first_tile + blockIdx.x) * kTile + threadIdx.x * 4u;
  const f32x4 x = ld(reinterpret_cast<const f32x4*>(a + i));
  const f32x4 y = ld(reinterpret_cast<const f32x4*>(b + i));
  st(reinterpret_cast<f32x4*>(a + i), x + s * y);
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" {

// 0 on success, 1 for arguments the kernels do not take (n not a multiple of 256, arrays not
// 16-byte aligned, replica count not 8, NULLs), 4 for a launch failure.
int zero_ceiling_twin(const void* const* reps, uint32_t nrep, uint64_t n, float* P, float* M,
                      float* V, void* out, float c, void* stream) {
  if (!reps || nrep != kReps || !P || !M || !V || !out || n % kTile != 0) return 1;
  Rows r{};
  for (int k = 0; k < kReps; ++k) {
    if (!reps[k] || !aligned(reps[k], 8)) return 1;
    r.p[k] = static_cast<const uint16_t*>(reps[k]);
  }
  if (!aligned(P, 16) || !aligned(M, 16) || !aligned(V, 16) || !aligned(out, 8)) return 1;
  const uint64_t tiles = n / kTile;
  (void)hipGetLastError();
  for (uint64_t t = 0; t < tiles; t += kMaxGrid) {
    const uint64_t g = tiles - t < kMaxGrid ? tiles - t : kMaxGrid;
    hipLaunchKernelGGL(k_twin, dim3((unsigned)g), dim3(64), 0, static_cast<hipStream_t>(stream), r,
                       t, P, M, V, static_cast<uint16_t*>(out), c);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int zero_ceiling_triad(float* a, const float* b, uint64_t n, float s, void* stream) {
  if (!a || !b || n % kTile != 0 || !aligned(a, 16) || !aligned(b, 16)) return 1;
  const uint64_t tiles = n / kTile;
  (void)hipGetLastError();
  for (uint64_t t = 0; t < tiles; t += kMaxGrid) {
    const uint64_t g = tiles - t < kMaxGrid ? tiles - t : kMaxGrid;
    hipLaunchKernelGGL(k_triad, dim3((unsigned)g), dim3(64), 0, static_cast<hipStream_t>(stream), a,
                       b, t, s);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // extern "C"

// gfx950 kernels of the per-rank sharded optimizer step and their C-ABI launchers.
//
// Everything here is HBM-bound elementwise streaming (about 0.5 flop per byte), so nothing is
// shaped for MFMA. A tile is SUB groups of 4 consecutive elements per thread, the groups spaced
// block*4 elements apart, so every load instruction of a wave covers one contiguous 1 KiB (fp32)
// or 512 B (16-bit) run. Loads and stores are non-temporal: every byte is touched once per step.
// The Adam kernel runs one single-wave tile per block over the aligned whole tiles of the shard,
// plus one block for a partial last tile; a separate per-element kernel takes arrays that are not
// 16-byte aligned.
// Measured on MI355X, one-wave blocks with one group per lane (a 256-element tile) moved this
// 15-stream read/write mix fastest: faster than 2 or 4 groups per lane, 128- or 256-thread blocks,
// grid-stride (persistent) launches and software-pipelined multi-tile blocks.
//
// Arithmetic is fp32 with every operation rounded on its own: the library is built with
// -ffp-contract=off and HIP's correctly rounded fp32 division and square root, so the results
// equal a plain IEEE evaluation of the same expression order bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <cmath>
#include <utility>

#include "zero_device.h"
#include "zero_internal.h"

#ifndef ZERO_ADAM_SUB
#define ZERO_ADAM_SUB 1            // 4-element groups per thread per tile in the Adam kernel
#endif
#ifndef ZERO_ADAM_BLOCK
#define ZERO_ADAM_BLOCK 64         // threads per block of the Adam kernel (one wave)
#endif
#ifndef ZERO_REP_BATCH
#define ZERO_REP_BATCH 8           // replica loads issued together before they are summed
#endif

namespace {

constexpr int kBlock = 256;            // the per-element tail kernels and the squared-norm finish
constexpr int kWaves = kBlock / 64;
constexpr int kAdamBlock = ZERO_ADAM_BLOCK;

using zero::f32x2;
using zero::f32x4;
using zero::ld;
using zero::st;
using zero::u32x2;

// f(0), f(1), ..., f(N-1) with compile-time indices and no loop in the code. A loop that runs
// once (N = 1) lets loop-invariant code motion promote its stores, and the promoted stores lose
// their non-temporal hint before the loop would be unrolled.
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

struct RepPtrs {
  const void* p[ZERO_MAX_REPLICAS];
};

struct StepScalars {
  float gs;  // grad_scale
  float b1, b2, c1, c2, ss, bc, e, dec, w;
};

// Step inputs that live in device memory: the grad scale (zero_clip_scale writes it) and,
// optionally, the step t with a table of per-step constants (entry t-1; t past the table takes
// its last entry).
struct DevCtl {
  const float* gs;
  const zero_adam_scalars* table;  // NULL: the constants passed in StepScalars
  const int64_t* step;
  uint32_t table_len;
};

__device__ __forceinline__ void dev_scalars(const DevCtl& dc, StepScalars& sc) {
  sc.gs = *dc.gs;
  if (dc.table != nullptr) {
    const int64_t t = *dc.step;
    const uint32_t i =
        t < 1 ? 0u : (t >= (int64_t)dc.table_len ? dc.table_len - 1u : (uint32_t)(t - 1));
    const zero_adam_scalars k = dc.table[i];
    sc.b1 = k.b1;
    sc.b2 = k.b2;
    sc.c1 = k.c1;
    sc.c2 = k.c2;
    sc.ss = k.ss;
    sc.bc = k.bc;
    sc.e = k.e;
    sc.dec = k.dec;
    sc.w = k.w;
  }
}

// ---------------------------------------------------------------------------------------------
// element conversions

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// fp32 -> 16-bit, round to nearest even, two values packed low-then-high. bf16 uses gfx950's
// v_cvt_pk_bf16_f32: checked against the integer rule (u + 0x7fff + ((u >> 16) & 1)) >> 16, with a
// NaN becoming (u >> 16) | 0x40, on all 2^32 fp32 patterns in the library's floating-point mode.
// binary16 uses the IEEE conversion in the default rounding mode.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <int ODT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 x = {a, b};
  if constexpr (ODT == ZERO_BF16) return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  else return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}

template <int ODT>
__device__ __forceinline__ uint16_t to_out1(float x) {
  if constexpr (ODT == ZERO_BF16) return __builtin_bit_cast(uint16_t, (__bf16)x);
  else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// 4 consecutive replica elements starting at element i (vector path: i is a multiple of 4 and
// the array is aligned to 4 elements).
template <int RDT>
__device__ __forceinline__ f32x4 ld_rep4(const void* base, uint64_t i) {
  if constexpr (RDT == ZERO_F32) {
    return ld(reinterpret_cast<const f32x4*>(static_cast<const float*>(base) + i));
  } else {
    const u32x2 w = ld(reinterpret_cast<const u32x2*>(static_cast<const uint16_t*>(base) + i));
    f32x4 r;
    if constexpr (RDT == ZERO_BF16) {
      r.x = __uint_as_float(w.x << 16);
      r.y = __uint_as_float(w.x & 0xffff0000u);
      r.z = __uint_as_float(w.y << 16);
      r.w = __uint_as_float(w.y & 0xffff0000u);
    } else {
      r.x = f16_to_f32(w.x & 0xffffu);
      r.y = f16_to_f32(w.x >> 16);
      r.z = f16_to_f32(w.y & 0xffffu);
      r.w = f16_to_f32(w.y >> 16);
    }
    return r;
  }
}

template <int RDT>
__device__ __forceinline__ float ld_rep1(const void* base, uint64_t i) {
  if constexpr (RDT == ZERO_F32) return static_cast<const float*>(base)[i];
  else if constexpr (RDT == ZERO_BF16) return bf16_to_f32(static_cast<const uint16_t*>(base)[i]);
  else return f16_to_f32(static_cast<const uint16_t*>(base)[i]);
}

// ---------------------------------------------------------------------------------------------
// replica sum: acc = rep_0 + rep_1 + ... in ascending order (loads issued 8 replicas at a time)

template <int RDT, int RFIX, int SUB>
__device__ __forceinline__ void sum_reps4(const RepPtrs& reps, int nrep, const uint64_t (&idx)[SUB],
                                          f32x4 (&acc)[SUB]) {
  constexpr int B = ZERO_REP_BATCH;   // replica loads in flight per lane before their adds
  const int R = RFIX ? RFIX : nrep;
#pragma unroll
  for (int u = 0; u < SUB; ++u) acc[u] = ld_rep4<RDT>(reps.p[0], idx[u]);
  for (int k0 = 1; k0 < R; k0 += B) {
    f32x4 t[B][SUB];
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (k0 + j < R) {
#pragma unroll
        for (int u = 0; u < SUB; ++u) t[j][u] = ld_rep4<RDT>(reps.p[k0 + j], idx[u]);
      }
#pragma unroll
    for (int j = 0; j < B; ++j)
      if (k0 + j < R) {
#pragma unroll
        for (int u = 0; u < SUB; ++u) acc[u] = acc[u] + t[j][u];
      }
  }
}

template <int RDT>
__device__ __forceinline__ float sum_reps1(const RepPtrs& reps, int nrep, uint64_t i) {
  float a = ld_rep1<RDT>(reps.p[0], i);
  for (int k = 1; k < nrep; ++k) a = a + ld_rep1<RDT>(reps.p[k], i);
  return a;
}

// ---------------------------------------------------------------------------------------------
// one element of Adam / AdamW, every operation rounded on its own

template <bool L2>
__device__ __forceinline__ void adam1(float acc, float& p, float& m, float& v, const StepScalars& s) {
  float g = acc * s.gs;
  if (L2) g = g + s.w * p;
  m = s.b1 * m + s.c1 * g;
  v = s.b2 * v + s.c2 * (g * g);
  const float den = sqrtf(v) / s.bc + s.e;
  if (!L2) p = p * s.dec;
  p = p - s.ss * (m / den);
}

// ---------------------------------------------------------------------------------------------
// fused step: replica sum -> Adam/AdamW on master/m/v -> 16-bit cast into the rank's slot
//
// Two kernels share the arithmetic. k_adam_step covers whole tiles of arrays that are all 16-byte
// aligned (8-byte for 16-bit arrays) with vector loads and stores, one tile per block. When the
// shard ends in a partial tile, the TAIL variant's grid has one block more, which walks that
// remainder (fewer than one tile) element by element, so a ragged shard still takes one launch.
// k_adam_tail covers the arrays that are not aligned, one element per thread.

// element i of the update: replica sum, Adam, 16-bit cast (any alignment)
template <int RDT, int ODT, bool L2>
__device__ __forceinline__ void adam_elem(const RepPtrs& reps, int nrep, uint64_t i,
                                          const StepScalars& sc, float* __restrict__ P,
                                          float* __restrict__ M, float* __restrict__ V,
                                          void* __restrict__ out) {
  const float a = sum_reps1<RDT>(reps, nrep, i);
  float p = P[i], m = M[i], v = V[i];
  adam1<L2>(a, p, m, v, sc);
  P[i] = p;
  M[i] = m;
  V[i] = v;
  if constexpr (ODT != ZERO_F32) static_cast<uint16_t*>(out)[i] = to_out1<ODT>(p);
}

template <int RDT, int ODT, bool L2, int RFIX, bool SKIP, bool TAIL, bool DGS>
__global__ __launch_bounds__(kAdamBlock) void k_adam_step(
    RepPtrs reps, int nrep, uint64_t first_tile, StepScalars sc, float* __restrict__ P,
    float* __restrict__ M, float* __restrict__ V, void* __restrict__ out,
    const int32_t* __restrict__ skip, DevCtl dc, uint64_t n) {
  // One tile per block and the grid is exactly the tile count (plus the remainder block with
  // TAIL): no loop bound and no per-block bound check to wait for, so a block's first loads issue
  // right after its arguments arrive.
  if constexpr (SKIP) {
    if (*skip != 0) return;
  }
  if constexpr (DGS) dev_scalars(dc, sc);   // grad scale (and step constants) from device memory
  constexpr uint64_t kTileElems = (uint64_t)kAdamBlock * 4 * ZERO_ADAM_SUB;
  if constexpr (TAIL) {
    if (blockIdx.x == gridDim.x - 1) {   // elements [tile start, n): fewer than one tile
#pragma unroll 1   // kept rolled: its registers must not raise the whole-tile path's budget
      for (uint64_t i = (first_tile + blockIdx.x) * kTileElems + threadIdx.x; i < n; i += kAdamBlock)
        adam_elem<RDT, ODT, L2>(reps, nrep, i, sc, P, M, V, out);
      return;
    }
  }
  constexpr int SUB = ZERO_ADAM_SUB;
  constexpr uint64_t kTile = (uint64_t)kAdamBlock * 4 * SUB;
  const uint64_t base = (first_tile + blockIdx.x) * kTile;
  uint64_t idx[SUB];
#pragma unroll
  for (int u = 0; u < SUB; ++u) idx[u] = base + (uint64_t)u * (kAdamBlock * 4) + threadIdx.x * 4u;
  f32x4 p[SUB], m[SUB], v[SUB], acc[SUB];
#pragma unroll
  for (int u = 0; u < SUB; ++u) {
    p[u] = ld(reinterpret_cast<const f32x4*>(P + idx[u]));
    m[u] = ld(reinterpret_cast<const f32x4*>(M + idx[u]));
    v[u] = ld(reinterpret_cast<const f32x4*>(V + idx[u]));
  }
  sum_reps4<RDT, RFIX, SUB>(reps, nrep, idx, acc);
  unroll<SUB>([&](auto u) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float pq = p[u][q], mq = m[u][q], vq = v[u][q];
      adam1<L2>(acc[u][q], pq, mq, vq, sc);
      p[u][q] = pq;
      m[u][q] = mq;
      v[u][q] = vq;
    }
    st(reinterpret_cast<f32x4*>(P + idx[u]), p[u]);
    st(reinterpret_cast<f32x4*>(M + idx[u]), m[u]);
    st(reinterpret_cast<f32x4*>(V + idx[u]), v[u]);
    if constexpr (ODT != ZERO_F32) {
      const u32x2 o = {pack2<ODT>(p[u].x, p[u].y), pack2<ODT>(p[u].z, p[u].w)};
      st(reinterpret_cast<u32x2*>(static_cast<uint16_t*>(out) + idx[u]), o);
    }
  });
}

// elements [begin, n), one per thread per grid-stride iteration, any alignment
template <int RDT, int ODT, bool L2>
__global__ __launch_bounds__(kBlock) void k_adam_tail(RepPtrs reps, int nrep, uint64_t begin,
                                                      uint64_t n, StepScalars sc,
                                                      float* __restrict__ P, float* __restrict__ M,
                                                      float* __restrict__ V, void* __restrict__ out,
                                                      const int32_t* __restrict__ skip,
                                                      DevCtl dc) {
  if (skip != nullptr && *skip != 0) return;
  if (dc.gs != nullptr) dev_scalars(dc, sc);
  for (uint64_t i = begin + (uint64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
       i += (uint64_t)gridDim.x * kBlock)
    adam_elem<RDT, ODT, L2>(reps, nrep, i, sc, P, M, V, out);
}

// ---------------------------------------------------------------------------------------------
// reduce pass: replica sum -> fp32 gradient, non-finite flag, fp64 squared-norm partials
//
// One single-wave block per tile of kRedTile = 256 elements, the Adam kernel's tile. Thread `lane`
// owns the elements base + u*256 + lane*4 + q (u < kRedSub, q < 4) and adds their fp64 squares in
// that (u, q) order; the 64 lane sums are combined by a fixed xor butterfly and lane 0 writes
// partial[tile]. On MI355X one group per lane (kRedSub = 1) took 2.4% less time for the 16-replica
// reduce than two groups and 4.7% less than four, as it does for the Adam kernel. The vector
// path (whole, aligned tiles) and the per-element path (ragged last tile, unaligned arrays) use
// the same element-to-lane map and order, so a partial never depends on alignment. The finish is
// a fixed two-level sum (zero_shard_sqnorm), so the squared norm is bit-reproducible for a given
// input and n. No atomics: the flag is only ever set to 1 by plain stores.

constexpr int kRedSub = 1;
constexpr uint64_t kRedTile = 64 * 4 * kRedSub;   // 256 elements
constexpr uint32_t kSqLevel1 = 1024;               // second-level partial slots

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;  // lane 0's value is the fixed-order result
}

__device__ __forceinline__ double block_sum(double x, double* lds) {
  x = wave_sum(x);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) lds[wave] = x;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
    s = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += lds[w];
  }
  return s;  // meaningful in thread 0 only
}

__device__ __forceinline__ bool nonfinite(float x) {
  return (__float_as_uint(x) & 0x7f800000u) == 0x7f800000u;
}

template <int RDT, int RFIX, bool VEC>
__device__ __forceinline__ void reduce_tile(const RepPtrs& reps, int nrep, uint64_t tile, uint64_t n,
                                            float* __restrict__ G, int32_t* __restrict__ flag,
                                            double* __restrict__ partials, double sq_scale) {
  const uint64_t base = tile * kRedTile;
  double sq = 0.0;
  bool bad = false;
  if constexpr (VEC) {
    uint64_t idx[kRedSub];
#pragma unroll
    for (int u = 0; u < kRedSub; ++u) idx[u] = base + (uint64_t)u * 256 + threadIdx.x * 4u;
    f32x4 acc[kRedSub];
    sum_reps4<RDT, RFIX, kRedSub>(reps, nrep, idx, acc);
    unroll<kRedSub>([&](auto u) {
      if (G != nullptr) st(reinterpret_cast<f32x4*>(G + idx[u]), acc[u]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bad |= nonfinite(acc[u][q]);
        const double d = (double)acc[u][q] * sq_scale;
        sq += d * d;
      }
    });
  } else {
    for (int u = 0; u < kRedSub; ++u)
      for (int q = 0; q < 4; ++q) {
        const uint64_t i = base + (uint64_t)u * 256 + threadIdx.x * 4u + q;
        if (i < n) {
          const float a = sum_reps1<RDT>(reps, nrep, i);
          if (G != nullptr) G[i] = a;
          bad |= nonfinite(a);
          const double d = (double)a * sq_scale;
          sq += d * d;
        }
      }
  }
  if (flag != nullptr && __ballot(bad) != 0 && threadIdx.x == 0) *flag = 1;
  if (partials != nullptr) {
    sq = wave_sum(sq);
    if (threadIdx.x == 0) partials[tile] = sq;
  }
}

// whole, aligned tiles with vector loads; with TAIL the grid has one block more, which takes the
// partial last tile element by element (same element order, so its partial is the same)
template <int RDT, int RFIX, bool TAIL>
__global__ __launch_bounds__(64) void k_reduce(RepPtrs reps, int nrep, uint64_t first_tile,
                                               uint64_t n, float* __restrict__ G,
                                               int32_t* __restrict__ flag,
                                               double* __restrict__ partials, double sq_scale) {
  if constexpr (TAIL) {
    if (blockIdx.x == gridDim.x - 1) {
      reduce_tile<RDT, 0, false>(reps, nrep, first_tile + blockIdx.x, n, G, flag, partials, sq_scale);
      return;
    }
  }
  reduce_tile<RDT, RFIX, true>(reps, nrep, first_tile + blockIdx.x, n, G, flag, partials, sq_scale);
}

// every tile of arrays that are not aligned: element by element
template <int RDT>
__global__ __launch_bounds__(64) void k_reduce_tail(RepPtrs reps, int nrep, uint64_t first_tile,
                                                    uint64_t n, float* __restrict__ G,
                                                    int32_t* __restrict__ flag,
                                                    double* __restrict__ partials, double sq_scale) {
  reduce_tile<RDT, 0, false>(reps, nrep, first_tile + blockIdx.x, n, G, flag, partials, sq_scale);
}

// level 1: block b sums partials [b*chunk, min(ntiles, (b+1)*chunk)) into partials[ntiles + b]
__global__ __launch_bounds__(kBlock) void k_sq_level1(double* __restrict__ partials, uint64_t ntiles,
                                                      uint64_t chunk) {
  __shared__ double lds[kWaves];
  const uint64_t lo = (uint64_t)blockIdx.x * chunk;
  const uint64_t hi = lo + chunk < ntiles ? lo + chunk : ntiles;
  double s = 0.0;
  for (uint64_t i = lo + threadIdx.x; i < hi; i += kBlock) s += partials[i];
  s = block_sum(s, lds);
  if (threadIdx.x == 0) partials[ntiles + blockIdx.x] = s;
}

// level 2: one block sums the `count` level-1 values at `l1` into *out
__global__ __launch_bounds__(kBlock) void k_sq_finalize(const double* __restrict__ l1,
                                                        uint32_t count, double* __restrict__ out) {
  __shared__ double lds[kWaves];
  double s = 0.0;
  for (uint32_t i = threadIdx.x; i < count; i += kBlock) s += l1[i];
  s = block_sum(s, lds);
  if (threadIdx.x == 0) *out = s;
}

// clip scale: q = max_norm / (sqrt(sq) + eps) in fp64, coef = min(1, q) (1 for a NaN q), and the
// fp32 grad scale coef * inv_loss_scale rounded to nearest even. fp64 division and square root are
// correctly rounded in this build, as on the host.
__global__ __launch_bounds__(64) void k_clip_scale(const double* __restrict__ sq, double max_norm,
                                                   double eps, double inv_loss_scale,
                                                   float* __restrict__ gs) {
  if (threadIdx.x != 0) return;
  const double q = max_norm / (sqrt(*sq) + eps);
  const double coef = q < 1.0 ? q : 1.0;
  *gs = (float)(coef * inv_loss_scale);
}

// the step counter after an update: t advances unless the update was skipped
__global__ __launch_bounds__(64) void k_step_advance(int64_t* __restrict__ step,
                                                     const int32_t* __restrict__ skip) {
  if (threadIdx.x != 0) return;
  if (skip == nullptr || *skip == 0) *step = *step + 1;
}

// ---------------------------------------------------------------------------------------------
// host side

constexpr int kMaxDevices = 64;
// per-device compute-unit count, filled on first use; threads that fill it at once store the same
// value, and the atomics make that well defined
std::atomic<int> g_cu_count[kMaxDevices];

zero_status cu_count(int* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return zero::fail(ZERO_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return zero::fail(ZERO_E_UNSUPPORTED, "device index %d", dev);
  int cached = g_cu_count[dev].load(std::memory_order_relaxed);
  if (cached == 0) {
    int cus = 0;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
      return zero::fail(ZERO_E_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    cached = cus > 0 ? cus : 1;
    g_cu_count[dev].store(cached, std::memory_order_relaxed);
  }
  *out = cached;
  return ZERO_OK;
}

zero_status launched(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return zero::fail(ZERO_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return zero::ok();
}

zero_status check_src(const char* fn, const zero_grad_src* src, uint64_t n) {
  if (!src || !src->ptrs) return zero::fail(ZERO_E_INVAL, "%s: gradient source is NULL", fn);
  if (src->count == 0 || src->count > ZERO_MAX_REPLICAS)
    return zero::fail(ZERO_E_INVAL, "%s: replica count %u outside 1..%d", fn, src->count,
                      ZERO_MAX_REPLICAS);
  if (!zero::dtype_valid(src->dtype))
    return zero::fail(ZERO_E_INVAL, "%s: unknown replica dtype %d", fn, src->dtype);
  for (uint32_t k = 0; k < src->count && n > 0; ++k)   // zero-length arrays may be NULL
    if (!src->ptrs[k]) return zero::fail(ZERO_E_INVAL, "%s: replica %u is NULL", fn, k);
  if (n > UINT64_MAX / 8) return zero::fail(ZERO_E_OVERFLOW, "%s: n = %llu too large", fn,
                                            (unsigned long long)n);
  return ZERO_OK;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool src_aligned(const zero_grad_src* src) {
  const uintptr_t a = 4u * zero::dtype_bytes(src->dtype);
  for (uint32_t k = 0; k < src->count; ++k)
    if (!aligned(src->ptrs[k], a)) return false;
  return true;
}

RepPtrs rep_ptrs(const zero_grad_src* src) {
  RepPtrs r{};
  for (uint32_t k = 0; k < src->count; ++k) r.p[k] = src->ptrs[k];
  return r;
}

// ----- Adam dispatch

constexpr uint64_t kAdamTile = (uint64_t)kAdamBlock * 4 * ZERO_ADAM_SUB;
constexpr uint64_t kMaxGrid = 1u << 24;  // blocks per Adam launch; keeps grid * block below 2^32

struct AdamArgs {
  RepPtrs reps;
  int nrep;
  uint64_t ntiles;      // whole vector tiles (k_adam_step), from element 0
  uint64_t tail_begin;  // first element of the per-element range (k_adam_tail)
  uint64_t n;
  StepScalars sc;
  float *P, *M, *V;
  void* out;
  const int32_t* skip;
  DevCtl dc;            // dc.gs == NULL: everything from sc
  unsigned tail_grid;
  hipStream_t stream;
  bool fused_tail;      // aligned shard with a partial last tile: k_adam_step's extra block takes it
};

template <int RDT, int ODT, bool L2, int RFIX, bool SKIP, bool TAIL>
void launch_adam_grid(const AdamArgs& a, uint64_t t0, uint64_t blocks) {
  if (a.dc.gs != nullptr)
    hipLaunchKernelGGL((k_adam_step<RDT, ODT, L2, RFIX, SKIP, TAIL, true>), dim3((unsigned)blocks),
                       dim3(kAdamBlock), 0, a.stream, a.reps, a.nrep, t0, a.sc, a.P, a.M, a.V,
                       a.out, a.skip, a.dc, a.n);
  else
    hipLaunchKernelGGL((k_adam_step<RDT, ODT, L2, RFIX, SKIP, TAIL, false>), dim3((unsigned)blocks),
                       dim3(kAdamBlock), 0, a.stream, a.reps, a.nrep, t0, a.sc, a.P, a.M, a.V,
                       a.out, a.skip, a.dc, a.n);
}

template <int RDT, int ODT, bool L2, int RFIX>
void launch_adam(const AdamArgs& a) {
  // Grids of at most kMaxGrid tiles, each told where its first tile is. A partial last tile of an
  // aligned shard rides on the last grid as one extra block (TAIL); a shard shorter than one tile
  // is then a grid of that block alone.
  const bool tail = a.fused_tail;
  uint64_t t0 = 0;
  do {
    const uint64_t g = a.ntiles - t0 < kMaxGrid ? a.ntiles - t0 : kMaxGrid;
    const bool last = t0 + g == a.ntiles;
    if (last && tail) {
      if (a.skip != nullptr) launch_adam_grid<RDT, ODT, L2, RFIX, true, true>(a, t0, g + 1);
      else launch_adam_grid<RDT, ODT, L2, RFIX, false, true>(a, t0, g + 1);
    } else if (g > 0) {
      if (a.skip != nullptr) launch_adam_grid<RDT, ODT, L2, RFIX, true, false>(a, t0, g);
      else launch_adam_grid<RDT, ODT, L2, RFIX, false, false>(a, t0, g);
    }
    t0 += g;
  } while (t0 < a.ntiles);
}

template <int RDT, int ODT, bool L2>
void adam_kernels(const AdamArgs& a) {
  if (a.ntiles > 0 || a.fused_tail) {
    switch (a.nrep) {
      case 1: launch_adam<RDT, ODT, L2, 1>(a); break;
      case 8: launch_adam<RDT, ODT, L2, 8>(a); break;
      case 16: launch_adam<RDT, ODT, L2, 16>(a); break;
      case 64: launch_adam<RDT, ODT, L2, 64>(a); break;
      default: launch_adam<RDT, ODT, L2, 0>(a); break;
    }
  }
  if (!a.fused_tail && a.tail_begin < a.n)
    hipLaunchKernelGGL((k_adam_tail<RDT, ODT, L2>), dim3(a.tail_grid), dim3(kBlock), 0, a.stream,
                       a.reps, a.nrep, a.tail_begin, a.n, a.sc, a.P, a.M, a.V, a.out, a.skip,
                       a.dc);
}

template <int RDT, int ODT>
void adam_by_l2(const AdamArgs& a, bool l2) {
  if (l2) adam_kernels<RDT, ODT, true>(a);
  else adam_kernels<RDT, ODT, false>(a);
}

template <int RDT>
void adam_by_out(const AdamArgs& a, int odt, bool l2) {
  if (odt == ZERO_BF16) adam_by_l2<RDT, ZERO_BF16>(a, l2);
  else if (odt == ZERO_F16) adam_by_l2<RDT, ZERO_F16>(a, l2);
  else adam_by_l2<RDT, ZERO_F32>(a, l2);  // ZERO_F32 here means "no 16-bit output"
}

// ----- reduce dispatch

uint64_t red_tiles(uint64_t n) { return n / kRedTile + (n % kRedTile != 0); }  // no wrap near 2^64

struct ReduceArgs {
  RepPtrs reps;
  int nrep;
  uint64_t n;
  float* G;
  int32_t* flag;
  double* partials;
  double sq_scale;
  hipStream_t stream;
};

// tiles [t0, t1) in grids of at most kMaxGrid blocks
// aligned arrays: tiles [0, full) as vector tiles in grids of at most kMaxGrid blocks; a partial
// last tile rides on the last grid as one extra block (a shard shorter than one tile is a grid of
// that block alone)
template <int RDT, int RFIX>
void launch_reduce_vec(const ReduceArgs& a, uint64_t full, bool tail) {
  uint64_t t = 0;
  do {
    const uint64_t g = full - t < kMaxGrid ? full - t : kMaxGrid;
    if (tail && t + g == full)
      hipLaunchKernelGGL((k_reduce<RDT, RFIX, true>), dim3((unsigned)(g + 1)), dim3(64), 0,
                         a.stream, a.reps, a.nrep, t, a.n, a.G, a.flag, a.partials, a.sq_scale);
    else if (g > 0)
      hipLaunchKernelGGL((k_reduce<RDT, RFIX, false>), dim3((unsigned)g), dim3(64), 0, a.stream,
                         a.reps, a.nrep, t, a.n, a.G, a.flag, a.partials, a.sq_scale);
    t += g;
  } while (t < full);
}

// arrays that are not aligned: every tile element by element, in grids of at most kMaxGrid
template <int RDT>
void launch_reduce_elem(const ReduceArgs& a, uint64_t tiles) {
  for (uint64_t t = 0; t < tiles; t += kMaxGrid) {
    const uint64_t g = tiles - t < kMaxGrid ? tiles - t : kMaxGrid;
    hipLaunchKernelGGL((k_reduce_tail<RDT>), dim3((unsigned)g), dim3(64), 0, a.stream, a.reps,
                       a.nrep, t, a.n, a.G, a.flag, a.partials, a.sq_scale);
  }
}

template <int RDT>
void reduce_kernels(const ReduceArgs& a, bool vec) {
  const uint64_t all = red_tiles(a.n);
  if (!vec) {
    launch_reduce_elem<RDT>(a, all);
    return;
  }
  const uint64_t full = a.n / kRedTile;
  const bool tail = all > full;
  switch (a.nrep) {
    case 1: launch_reduce_vec<RDT, 1>(a, full, tail); break;
    case 8: launch_reduce_vec<RDT, 8>(a, full, tail); break;
    case 16: launch_reduce_vec<RDT, 16>(a, full, tail); break;
    case 64: launch_reduce_vec<RDT, 64>(a, full, tail); break;
    default: launch_reduce_vec<RDT, 0>(a, full, tail); break;
  }
}

zero_status reduce_impl(const zero_grad_src* src, uint64_t n, float* G, int32_t* flag,
                        double* partials, double sq_scale, hipStream_t stream, const char* what) {
  if (n == 0) return zero::ok();
  ReduceArgs a{rep_ptrs(src), (int)src->count, n, G, flag, partials, sq_scale, stream};
  const bool vec = src_aligned(src) && (G == nullptr || aligned(G, 16));
  (void)hipGetLastError();
  switch (src->dtype) {
    case ZERO_F32: reduce_kernels<ZERO_F32>(a, vec); break;
    case ZERO_F16: reduce_kernels<ZERO_F16>(a, vec); break;
    default: reduce_kernels<ZERO_BF16>(a, vec); break;
  }
  return launched(what);
}

zero_status sq_finish(uint64_t n, double* partials, double* out, hipStream_t stream, const char* what) {
  const uint64_t ntiles = red_tiles(n);
  const uint32_t g1 = ntiles < kSqLevel1 ? (uint32_t)ntiles : kSqLevel1;
  (void)hipGetLastError();
  if (g1 > 0) {
    const uint64_t chunk = (ntiles + g1 - 1) / g1;
    hipLaunchKernelGGL(k_sq_level1, dim3(g1), dim3(kBlock), 0, stream, partials, ntiles, chunk);
  }
  hipLaunchKernelGGL(k_sq_finalize, dim3(1), dim3(kBlock), 0, stream, partials + ntiles, g1, out);
  return launched(what);
}

}  // namespace

extern "C" {

uint64_t zero_sq_partials_len(uint64_t n) { return red_tiles(n) + kSqLevel1; }

zero_status zero_reduce_shard(const zero_grad_src* src, uint64_t n, float* out_grad,
                              int32_t* d_nonfinite, double* d_sq_partials, double sq_scale,
                              void* stream) {
  const char* fn = "zero_reduce_shard";
  zero_status s = check_src(fn, src, n);
  if (s != ZERO_OK) return s;
  if (!out_grad && !d_nonfinite && !d_sq_partials)
    return zero::fail(ZERO_E_INVAL, "%s: no output requested", fn);
  const uint64_t rb = n * zero::dtype_bytes(src->dtype), pb = zero_sq_partials_len(n) * 8;
  for (uint32_t k = 0; k < src->count; ++k) {
    if (out_grad && zero::overlaps(out_grad, n * 4, src->ptrs[k], rb))
      return zero::fail(ZERO_E_INVAL, "%s: out_grad overlaps replica %u", fn, k);
    if (d_sq_partials && zero::overlaps(d_sq_partials, pb, src->ptrs[k], rb))
      return zero::fail(ZERO_E_INVAL, "%s: partials overlap replica %u", fn, k);
  }
  if (d_sq_partials && out_grad && zero::overlaps(d_sq_partials, pb, out_grad, n * 4))
    return zero::fail(ZERO_E_INVAL, "%s: partials overlap out_grad", fn);
  return reduce_impl(src, n, out_grad, d_nonfinite, d_sq_partials, sq_scale,
                     static_cast<hipStream_t>(stream), fn);
}

zero_status zero_shard_sqnorm(const float* d_grad, uint64_t n, double sq_scale, double* d_partials,
                              double* d_out, void* stream) {
  const char* fn = "zero_shard_sqnorm";
  if (!d_partials || !d_out) return zero::fail(ZERO_E_INVAL, "%s: partials or out is NULL", fn);
  if (n > UINT64_MAX / 8)
    return zero::fail(ZERO_E_OVERFLOW, "%s: n = %llu too large", fn, (unsigned long long)n);
  const uint64_t pb = zero_sq_partials_len(n) * 8;
  if (zero::overlaps(d_partials, pb, d_out, 8))
    return zero::fail(ZERO_E_INVAL, "%s: out overlaps the partials", fn);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d_grad != nullptr) {
    const void* ptrs[1] = {d_grad};
    const zero_grad_src src{ptrs, 1, ZERO_F32};
    zero_status s = check_src(fn, &src, n);
    if (s != ZERO_OK) return s;
    if (zero::overlaps(d_partials, pb, d_grad, n * 4))
      return zero::fail(ZERO_E_INVAL, "%s: partials overlap the gradient", fn);
    if (zero::overlaps(d_out, 8, d_grad, n * 4))
      return zero::fail(ZERO_E_INVAL, "%s: out overlaps the gradient", fn);
    s = reduce_impl(&src, n, nullptr, nullptr, d_partials, sq_scale, st, fn);
    if (s != ZERO_OK) return s;
  }
  return sq_finish(n, d_partials, d_out, st, fn);
}

}  // extern "C"

namespace {

// every step entry point: constants in sc0, or from device memory as dc says (dc.gs != NULL)
zero_status adam_step_impl(const char* fn, const zero_grad_src* src, uint64_t n,
                           const StepScalars& sc0, const DevCtl& dc, bool l2, float* master,
                           float* m, float* v, void* out_param, int32_t out_dtype,
                           const int32_t* d_skip, void* stream) {
  zero_status s = check_src(fn, src, n);
  if (s != ZERO_OK) return s;
  if (n > 0 && (!master || !m || !v))
    return zero::fail(ZERO_E_INVAL, "%s: master, m or v is NULL", fn);
  if (out_param) {
    if (out_dtype == ZERO_F32)
      return zero::fail(ZERO_E_UNSUPPORTED, "%s: fp32 parameter output is not supported", fn);
    if (out_dtype != ZERO_BF16 && out_dtype != ZERO_F16)
      return zero::fail(ZERO_E_INVAL, "%s: unknown out dtype %d", fn, out_dtype);
  }
  const uint64_t sb = n * 4, ob = out_param ? n * 2 : 0, rb = n * zero::dtype_bytes(src->dtype);
  const void* own[4] = {master, m, v, out_param};
  const uint64_t own_b[4] = {sb, sb, sb, ob};
  // device inputs the update reads (grad scale, constants table, step) must not be written by it
  const void* dev_in[3] = {dc.gs, dc.table, dc.step};
  const uint64_t dev_in_b[3] = {dc.gs ? 4u : 0u, dc.table ? (uint64_t)dc.table_len * sizeof(zero_adam_scalars) : 0u,
                                dc.step ? 8u : 0u};
  for (int x = 0; x < 4; ++x) {
    for (int y = x + 1; y < 4; ++y)
      if (zero::overlaps(own[x], own_b[x], own[y], own_b[y]))
        return zero::fail(ZERO_E_INVAL, "%s: output arrays %d and %d overlap", fn, x, y);
    for (uint32_t r = 0; r < src->count; ++r)
      if (zero::overlaps(own[x], own_b[x], src->ptrs[r], rb))
        return zero::fail(ZERO_E_INVAL, "%s: output array %d overlaps replica %u", fn, x, r);
    for (int d = 0; d < 3; ++d)
      if (zero::overlaps(own[x], own_b[x], dev_in[d], dev_in_b[d]))
        return zero::fail(ZERO_E_INVAL, "%s: output array %d overlaps the %s", fn, x,
                          d == 0 ? "grad scale" : d == 1 ? "constants table" : "step");
  }
  if (n == 0) return zero::ok();

  int cus = 0;
  s = cu_count(&cus);
  if (s != ZERO_OK) return s;
  const bool vec = src_aligned(src) && aligned(master, 16) && aligned(m, 16) && aligned(v, 16) &&
                   (out_param == nullptr || aligned(out_param, 8));
  const uint64_t ntiles = vec ? n / kAdamTile : 0;
  const uint64_t tail_begin = ntiles * kAdamTile, tail_n = n - tail_begin;
  uint64_t tail_grid = (tail_n + kBlock - 1) / kBlock;
  if (tail_grid > (uint64_t)cus * 8) tail_grid = (uint64_t)cus * 8;
  AdamArgs a{rep_ptrs(src), (int)src->count, ntiles, tail_begin, n, sc0,
             master, m, v, out_param, d_skip, dc, (unsigned)tail_grid,
             static_cast<hipStream_t>(stream), vec && tail_n > 0};
  const int odt = out_param ? out_dtype : ZERO_F32;
  (void)hipGetLastError();
  switch (src->dtype) {
    case ZERO_F32: adam_by_out<ZERO_F32>(a, odt, l2); break;
    case ZERO_F16: adam_by_out<ZERO_F16>(a, odt, l2); break;
    default: adam_by_out<ZERO_BF16>(a, odt, l2); break;
  }
  return launched(fn);
}

// the host-step entry points: constants derived from hp on the host
zero_status adam_step_host_t(const char* fn, const zero_grad_src* src, uint64_t n,
                             float grad_scale, const float* d_grad_scale, float* master, float* m,
                             float* v, const zero_adam_hparams* hp, void* out_param,
                             int32_t out_dtype, const int32_t* d_skip, void* stream) {
  zero_adam_scalars k;
  const zero_status s = zero_adam_derive(hp, &k);
  if (s != ZERO_OK) return s;
  const StepScalars sc{grad_scale, k.b1, k.b2, k.c1, k.c2, k.ss, k.bc, k.e, k.dec, k.w};
  const DevCtl dc{d_grad_scale, nullptr, nullptr, 0};
  return adam_step_impl(fn, src, n, sc, dc, hp->wd_mode == ZERO_ADAM_L2, master, m, v, out_param,
                        out_dtype, d_skip, stream);
}

}  // namespace

extern "C" {

zero_status zero_adam_shard_step(const zero_grad_src* src, uint64_t n, float grad_scale,
                                 float* master, float* m, float* v, const zero_adam_hparams* hp,
                                 void* out_param, int32_t out_dtype, const int32_t* d_skip,
                                 void* stream) {
  return adam_step_host_t("zero_adam_shard_step", src, n, grad_scale, nullptr, master, m, v, hp,
                          out_param, out_dtype, d_skip, stream);
}

zero_status zero_adam_shard_step_dev_scale(const zero_grad_src* src, uint64_t n,
                                           const float* d_grad_scale, float* master, float* m,
                                           float* v, const zero_adam_hparams* hp, void* out_param,
                                           int32_t out_dtype, const int32_t* d_skip,
                                           void* stream) {
  const char* fn = "zero_adam_shard_step_dev_scale";
  if (!d_grad_scale) return zero::fail(ZERO_E_INVAL, "%s: d_grad_scale is NULL", fn);
  return adam_step_host_t(fn, src, n, 1.0f, d_grad_scale, master, m, v, hp, out_param, out_dtype,
                          d_skip, stream);
}

zero_status zero_adam_shard_step_dev_t(const zero_grad_src* src, uint64_t n,
                                       const float* d_grad_scale, const zero_adam_scalars* d_table,
                                       uint32_t table_len, int64_t* d_step, int32_t wd_mode,
                                       float* master, float* m, float* v, void* out_param,
                                       int32_t out_dtype, const int32_t* d_skip, void* stream) {
  const char* fn = "zero_adam_shard_step_dev_t";
  if (!d_grad_scale || !d_table || !d_step)
    return zero::fail(ZERO_E_INVAL, "%s: d_grad_scale, d_table or d_step is NULL", fn);
  if (table_len == 0) return zero::fail(ZERO_E_INVAL, "%s: empty constants table", fn);
  if (wd_mode != ZERO_ADAMW && wd_mode != ZERO_ADAM_L2)
    return zero::fail(ZERO_E_INVAL, "%s: unknown wd_mode %d", fn, wd_mode);
  const uint64_t tb = (uint64_t)table_len * sizeof(zero_adam_scalars);
  if (zero::overlaps(d_step, 8, d_table, tb) || zero::overlaps(d_step, 8, d_grad_scale, 4) ||
      (d_skip && zero::overlaps(d_step, 8, d_skip, 4)))
    return zero::fail(ZERO_E_INVAL, "%s: d_step overlaps the table, the grad scale or the flag", fn);
  const StepScalars sc{1.0f, 0, 0, 0, 0, 0, 0, 0, 0, 0};   // all read from the table
  const DevCtl dc{d_grad_scale, d_table, d_step, table_len};
  zero_status s = adam_step_impl(fn, src, n, sc, dc, wd_mode == ZERO_ADAM_L2, master, m, v,
                                 out_param, out_dtype, d_skip, stream);
  if (s != ZERO_OK) return s;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_step_advance, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), d_step,
                     d_skip);
  return launched(fn);
}

zero_status zero_clip_scale(const double* d_sq, double max_norm, double clip_eps,
                            double inv_loss_scale, float* d_grad_scale, void* stream) {
  const char* fn = "zero_clip_scale";
  if (!d_sq || !d_grad_scale) return zero::fail(ZERO_E_INVAL, "%s: d_sq or d_grad_scale is NULL", fn);
  if (zero::overlaps(d_sq, 8, d_grad_scale, 4))
    return zero::fail(ZERO_E_INVAL, "%s: d_grad_scale overlaps d_sq", fn);
  if (!(std::isfinite(max_norm) && max_norm > 0.0))
    return zero::fail(ZERO_E_INVAL, "%s: max_norm %g is not finite and positive", fn, max_norm);
  if (!(std::isfinite(clip_eps) && clip_eps >= 0.0))
    return zero::fail(ZERO_E_INVAL, "%s: clip_eps %g is not finite and non-negative", fn, clip_eps);
  if (!(std::isfinite(inv_loss_scale) && inv_loss_scale > 0.0))
    return zero::fail(ZERO_E_INVAL, "%s: inv_loss_scale %g is not finite and positive", fn,
                      inv_loss_scale);
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_clip_scale, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), d_sq,
                     max_norm, clip_eps, inv_loss_scale, d_grad_scale);
  return launched(fn);
}

}  // extern "C"
